// Fused attention kernels for gfx950 (MI355X).
//
// One workgroup = 4 waves, one per SIMD.  Rows are "packed" grouped-query
// rows: packed row r of KV head hk is query position r / G of query head
// hk * G + r % G, so the G query heads that share a KV head sit in one
// workgroup and every K/V tile is staged into LDS once for all of them.
// At head_dim 256 a wave owns 32 packed rows and all columns (128 rows per
// workgroup, 64-key tiles); at 512 two waves share 32 rows and split the
// columns (64 rows per workgroup, 32-key tiles).
//
// Per K/V tile each wave computes, with 32x32x16 MFMAs,
//   S^T = K Q^T            (A = K rows from LDS, B = Q from registers)
//   online softmax         (one query row per lane pair, fp32, base 2)
//   O^T += V^T P^T         (A = V^T by transposing LDS reads, B = P from registers)
// Working with the transposed products keeps every row's scores, softmax
// state and output accumulator inside the two lanes that own the row, so
// the row max needs a single cross-lane exchange and the rescale of O is
// lane-local.  The score matrix never exists outside registers.
//
// This is the fused "tile K/V so it scales" kernel whose absence at
// head_dim 256 forces the materialized-score fallback in lablup/mlxcel issue
// #672 (Root cause) and that ml-explore/mlx PR #3293 instantiates for
// head_dim 256 (Changes, Routing update).  Its tile shapes are chosen for
// gfx950's 160 KiB LDS and 512-entry register file, not taken from the
// 32x16xBD Metal tiles discussed there (Analysis section).
#include "sdpa_internal.h"

#include <math.h>

#include <type_traits>

namespace sdpa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <int DT>
struct Elem;

template <>
struct Elem<0> {  // IEEE binary16
  static __device__ __forceinline__ f32x16_t mfma(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    // one v_cvt_pk_f16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
  }
  // acc + lo + hi of a packed pair, in fp32 (one v_dot2_f32_f16 against 1, 1)
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), (f16x2_t){1.0f16, 1.0f16}, acc, false);
  }
};

template <>
struct Elem<1> {  // bfloat16
  static __device__ __forceinline__ f32x16_t mfma(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    // one v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
  }
  // acc + lo + hi of a packed pair, in fp32 (one v_dot2_f32_bf16 against 1, 1)
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), (bf16x2_t){1.0f, 1.0f}, acc, false);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposing LDS read (ds_read_b64_tr_b16).  In each 16-lane group, source
// lane a + 4 t (a, t in 0..3) names 4 consecutive 16-bit elements of row t
// of a 4-row block; result lane 4 a' + b' receives element b' of the source
// lanes a' + 4 t for t = 0..3.  So when source lane a + 4 t points at V row
// (key0 + t), columns d0 + 4 a .. + 3, result lane j of the group holds keys
// key0 .. key0 + 3 of column d0 + j: a V^T operand slice, read straight from
// the key-major V tile.
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
__device__ __forceinline__ uint2 read_tr(const uint16_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)p));
}

// One 16-byte-per-lane direct load into LDS through a buffer descriptor:
// lane l reads the 16 bytes at base + voff and writes them to lds + 16 l.
// base, nbytes and lds are uniform.  A lane whose voff is nbytes or more is
// out of the descriptor's range: the hardware reads zeros for it instead of
// touching memory, so rows past the end of a K/V slab arrive as zeros with
// no per-lane clamp.  Issued through inline assembly so that the compiler
// does not treat it as a pending LDS write and wait for it before every
// later LDS access; the kernel waits for these loads itself, before the
// barrier that publishes the tile they fill.  M0 (the LDS base of the
// instruction) is restored afterwards; writing M0 needs one wait state
// before the load.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
// descriptor word 3 for untyped loads on gfx9-family GPUs: data format 32,
// no index stride, no swizzle
constexpr int kRsrcWord3 = 0x00020000;

// The 64-bit address of a uniform pointer in scalar registers (readfirstlane
// returns int, so each half goes through uint32_t: no sign extension).
__device__ __forceinline__ uint64_t uniform_addr(const void* ptr) {
  const uint64_t a = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// A uniform 64-bit value in a scalar register pair.
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Descriptor of `bytes` bytes from `base` (a uniform_addr value); word 1
// holds address bits 32..47 and a zero stride.
__device__ __forceinline__ i32x4_t tile_rsrc(uint64_t base, int bytes) {
  return i32x4_t{(int)(uint32_t)base, (int)((uint32_t)(base >> 32) & 0xffffu), bytes, kRsrcWord3};
}

// M0 holds the LDS base of a direct load.  No code the compiler generates
// for these kernels reads or writes M0 (a host test checks the generated
// assembly), so a run of loads saves M0 once, sets it per load and restores
// it after the last one.
__device__ __forceinline__ unsigned m0_save() {
  unsigned s;
  asm volatile("s_mov_b32 %0, m0" : "=s"(s));
  return s;
}
__device__ __forceinline__ void m0_restore(unsigned s) { asm volatile("s_mov_b32 m0, %0" ::"s"(s)); }

// Call between m0_save and m0_restore.  Lane l reads base + soff + voff
// (soff uniform) and is out of range when soff + voff reaches the
// descriptor's byte count.  Writing M0 needs one wait state before the
// load.
__device__ __forceinline__ void load_lds16(i32x4_t rsrc, uint32_t voff, uint32_t soff, void* lds) {
  const unsigned m0v = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds);
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff),
      "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)), "s"(m0v));
}

// The same with M0 = m0base + m0off formed in the asm: the constant m0off
// needs no register of its own between loads (the compiler re-creates a
// constant instead of keeping it), and only one base per buffer stays live.
__device__ __forceinline__ void load_lds16_off(i32x4_t rsrc, uint32_t voff, uint32_t soff, unsigned m0base,
                                               unsigned m0off) {
  asm volatile(
      "s_add_u32 m0, %3, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff),
      "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)), "s"(m0base), "s"(m0off)
      : "scc");
}

// Loads of four consecutive 1 KiB blocks share one M0 value: the load's
// immediate offset moves its LDS destination (M0 + offset + 16 lane) and
// its source (base + soff + voff + offset) together, and the range check
// covers voff + soff + offset.  Load k of a group (k = 0..3) takes offset
// 1024 k; load 0 writes M0 (m0base + m0off) first.  Nothing between the
// loads of a group may write M0.
template <int K>
__device__ __forceinline__ void load_lds16_grp(i32x4_t rsrc, uint32_t voff, uint32_t soff, unsigned m0base,
                                               unsigned m0off) {
  if constexpr (K == 0) {
    asm volatile(
        "s_add_u32 m0, %3, %4\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff),
        "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)), "s"(m0base), "s"(m0off)
        : "scc");
  } else {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds" ::"v"(voff), "s"(rsrc),
                 "s"(__builtin_amdgcn_readfirstlane(soff)), "i"(1024 * K));
  }
}

// The same for a block whose rows lie on both sides of the end of a ring of
// cache rows: the lanes in exec_a read through ra, the lanes in exec_b
// (the complement) through rb.  A lane outside the exec mask of a load
// neither reads memory nor writes LDS in it, so each lane is served by
// exactly one of the two loads.  EXEC is restored before the block ends.
__device__ __forceinline__ void load_lds16_2(i32x4_t ra, i32x4_t rb, uint64_t exec_a, uint64_t exec_b,
                                             uint32_t voff, uint32_t soff, uint32_t m0v) {
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_mov_b64 exec, %3\n\t"
      "s_nop 1\n\t"
      "buffer_load_dwordx4 %1, %2, %6 offen lds\n\t"
      "s_mov_b64 exec, %4\n\t"
      "s_nop 1\n\t"
      "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(ra), "s"(exec_a), "s"(exec_b), "s"(rb), "s"(__builtin_amdgcn_readfirstlane(soff)),
        "s"(m0v));
}

// (m & x) | (~m & y) bit by bit, one v_bfi_b32 (the compiler does not form
// it from the and/or expression).
__device__ __forceinline__ float bit_select(int m, float x, uint32_t y) {
  float r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(x), "s"(y));
  return r;
}

// max(a, b, c) in one v_max3_f32.  fmaxf on values the compiler cannot prove
// canonical gets extra self-max ops to quiet signalling NaNs; the scores
// here are finite or -inf (garbage only in the discarded step after the
// last tile), so they need none.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Max and sum over the two lanes (l, l ^ 32) that share a query row.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v),
                                                  __builtin_bit_cast(int, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v),
                                                  __builtin_bit_cast(int, v), false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Wait until at most N vector memory operations of this wave are
// outstanding (vmcnt only; LDS and export counters untouched).  Loads
// complete in issue order, so this waits for everything but the N most
// recent loads.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// K/V tiles of LDS per workgroup: 2 K + 3 V for the 256-wide LDS rows
// (head dims 192 and 256) without a bias tile, else 2 + 2 (the narrower
// rows keep two workgroups per CU within 256 registers)
constexpr int kv_tiles(bool bias, int dk) { return (!bias && dk > 128 && dk != 512) ? 5 : 4; }

// Lazy rescaling: a row's reference max moves only when a tile's max exceeds
// it by more than this many binary orders of magnitude, so exp2 arguments stay
// <= kRescaleLog2 (weights <= 256, well inside the fp16/bf16 range) and the
// output accumulator is rescaled only on those rare tiles.  The result is the
// same softmax; only rounding differs.
constexpr float kRescaleLog2 = 8.f;

// ---------------------------------------------------------------------------
// The attention kernel body: one wave per SIMD, 32 x 256 fp32 output
// accumulators per wave, software pipelined over K/V tiles.  While the MFMAs
// of S(t+1) = K(t+1) Q^T run, the same wave computes exp / sum / pack of
// tile t and issues the direct loads of the tiles after; while the MFMAs of
// O += P(t) V(t) run, it masks and takes the row max of S(t+1).  MFMAs and
// the vector work between them are independent, so the matrix unit keeps
// busy through the softmax.  K and V have separate double buffers, V one
// tile behind K: step t reads K(t+1) and V(t) and loads K(t+2) and V(t+1).
// ---------------------------------------------------------------------------
template <int DT, int DK, int DV, bool RING, bool BIAS, int Q4M = 0, bool PERS = false>
__device__ __forceinline__ void attn_pipe_body(const AttnParams& p, uint16_t* lds) {
  // PERS: the workgroup runs several row blocks of one (batch, KV head) with
  // one software pipeline (see the persistent loop below)
  // Q4M: 0 for 16-bit K/V; 4-bit K/V with 1: one row-holding wave (at most 32
  // packed rows: decode and verify steps), the other three load; 2: the
  // general instance (prefill over a 4-bit prefix), in which every wave loads
  // its share unless the workgroup has a single row-holding wave.  The host
  // picks the instance from the packed row count; the decode instance holds
  // only its own loaders' registers.
  constexpr bool Q4 = Q4M != 0;
  // DK: head dim of q and k; DV: head dim of v and the output.
  // DK <= 256: a wave owns 32 rows and all DV output columns.  DK = DV =
  // 512: the two waves of a pair own the same 32 rows; wave h multiplies Q
  // columns [256 h, 256 h + 256) into partial scores, the pair swaps them
  // through LDS and adds them (a + b == b + a: both hold bitwise identical
  // scores and run identical softmax arithmetic), and wave h accumulates
  // output columns [256 h, 256 h + 256).  Up to 32 x 256 fp32 accumulators
  // per wave.
  constexpr bool PAIR = (DK == 512);
  // MT: the 16-bit type of the staged K/V tiles, Q, P and the MFMAs.  The
  // input type, except for 4-bit K/V: there the dequantized elements are
  // staged as fp16 whatever the input type, since fp16 keeps 11 significant
  // bits to bf16's 8; a bf16 Q converts to fp16 exactly (for values inside
  // fp16's range), and the output is still rounded to the input type.
  constexpr int MT = Q4 ? 0 : DT;
  using EM = Elem<MT>;
  // V3: a third V buffer; V loaded in the P V region (see the step below)
  constexpr bool V3 = !Q4 && kv_tiles(BIAS, DK) == 5;
  // Q4: 4-bit K and V, dequantized into the same LDS tiles through registers
  static_assert(!Q4 || (DK == 256 && DV == 256 && !RING && !BIAS), "4-bit K/V: head dim 256 only");
  constexpr bool VLATE = PAIR || V3;
  constexpr int NVB = V3 ? 3 : 2;
  // GRP (D = 512 without a ring or bias): each wave loads contiguous 1 KiB
  // blocks of a tile, four to an M0 value (load_lds16_grp).  The K and the V
  // loads of a step each run in a region of their own, and a block is one
  // key row both in LDS and in memory.  (At D = 256 the same grouping gave
  // the same times.)
  constexpr bool GRP = PAIR && !RING && !BIAS;
  static_assert(PAIR == (DV == 512), "head dim 512 only with DK == DV");
  constexpr int NW = 4, RBW = PAIR ? 2 : 4;  // 32-row blocks per workgroup
  constexpr int BM = RBW * kRowsPerWave, BN = tile_keys(DK), KB = BN / 32;
  constexpr int DQ = DK < 256 ? DK : 256, DO = PAIR ? DV / 2 : DV;  // Q columns multiplied, output columns owned
  // output column blocks of 32: a head dim of 80 takes three, the last one
  // half beyond the value rows (their LDS columns read zeros, and the
  // epilogue writes only columns below DV)
  constexpr int DC = DQ / 16, DB = (DO + 31) / 32;
  static_assert(DQ % 16 == 0 && DO % 16 == 0, "head dims are multiples of 16");
  // K and V tiles sit in LDS as BN rows of LD elements; a head dim below LD
  // (192) leaves the end of each row unused, so that 192-wide rows take the
  // 256-wide layout and its swizzles unchanged
  constexpr int LD = lds_row(DK, DV);
  constexpr int ROWCH = LD / 8, TILE = BN * LD, LOADS = TILE * 2 / 1024 / NW;
  // score elements per lane; the S region has NQK MFMA slots and the P V
  // region NPV, each taking one or two of the elements' vector work
  constexpr int NE = KB * 16, NQK = KB * DC, NPV = KB * 2 * DB;
  // V rows of 16 chunks (LD = 128) swizzle over 4 rows, wider ones over 8
  constexpr int VSW = ROWCH >= 32 ? 7 : 3;
  static_assert(BM == block_rows(DK), "geometry");
  static_assert(LOADS == 4 || LOADS == 8, "K and V loads of 1 KiB blocks per wave");
  static_assert(NQK <= NE && NE <= 4 * NQK && NPV <= NE && NE <= 4 * NPV, "one to four score elements per MFMA slot");
  // the first score element of S slot n and of P V slot n (n <= the slot count)
  auto es = [](int n) { return (n < NQK ? n : NQK) * NE / NQK; };
  auto ev = [](int n) { return (n < NPV ? n : NPV) * NE / NPV; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int rb = PAIR ? (wave >> 1) : wave;  // this wave's 32-row block
  const int h = PAIR ? (wave & 1) : 0;       // this wave's half of the pair's work
  const int qd0 = h * DQ * (PAIR ? 1 : 0);   // first Q column this wave multiplies
  const int od0 = h * DO;                    // first output column this wave owns

  const int nheads = p.B * p.Hkv;
  // Workgroups are handed to the 8 XCDs round-robin by their linear index,
  // and each XCD has its own L2.  With p.xcd_heads the index maps so that an
  // XCD runs its heads one after another (all its workgroups on one head,
  // heaviest row blocks first), so each K/V tile fetched into its L2 serves
  // every workgroup of the head there; otherwise consecutive indices take
  // consecutive heads.
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int head = p.xcd_heads ? xcd + 8 * (slot / p.mblocks) : (int)(blockIdx.x % nheads);
  const int mbr = p.xcd_heads ? slot % p.mblocks : (int)(blockIdx.x / nheads);
  // PERS: workgroup w of a head runs row blocks w, w + S, w + 2 S, ... (S =
  // p.pers_stride workgroups per head), so that the workgroups that run at
  // the same time on an XCD work on neighbouring blocks and share K/V tiles
  // through its L2, as separate workgroups would
  const int mb = PERS ? mbr : p.causal ? (p.mblocks - 1 - mbr) : mbr;
  const int split = blockIdx.y;
  const int b = head / p.Hkv, hkv = head % p.Hkv;

  // the rows of row block mb: this wave's, this lane's, and the key range
  // they see (mutable only in the persistent loop, which moves to the next
  // block)
  int row0, rows_end, wrow0, my, qi, hq, pos, wp_lo, wp_hi;
  bool wave_active, valid;
  auto set_rows = [&](int mbx) {
    row0 = mbx * BM;
    rows_end = min(p.rows, row0 + BM);
    wrow0 = row0 + rb * kRowsPerWave;
    wave_active = wrow0 < rows_end;
    my = wrow0 + lr;
    valid = my < rows_end;
    qi = valid ? my / p.G : 0;
    hq = hkv * p.G + (valid ? my % p.G : 0);
    pos = p.q_offset + qi;
    // first and last query position of the wave's rows (uniform; scalar
    // registers, so that tile tests on them are scalar branches)
    wp_lo = __builtin_amdgcn_readfirstlane(p.q_offset + wrow0 / p.G);
    wp_hi = __builtin_amdgcn_readfirstlane(p.q_offset + (min(rows_end, wrow0 + kRowsPerWave) - 1) / p.G);
  };
  set_rows(mb);
  // the tiles row block mbx's rows see (within this split)
  auto block_keys = [&](int mbx, int& kb0, int& ke0) {
    const int r0 = mbx * BM, re = min(p.rows, r0 + BM);
    const int bp_lo = p.q_offset + r0 / p.G;
    const int bp_hi = p.q_offset + (re - 1) / p.G;
    kb0 = 0;
    ke0 = p.kL;
    if (p.causal) ke0 = min(ke0, bp_hi + 1);
    if (p.window > 0) kb0 = max(0, bp_lo - p.window + 1);
    if (p.partials) {
      kb0 = max(kb0, split * p.split_len);
      ke0 = min(ke0, (split + 1) * p.split_len);
    }
  };
  int kbeg, kend;
  block_keys(mb, kbeg, kend);
  if (kbeg >= kend) return;
  int t_first = __builtin_amdgcn_readfirstlane(kbeg / BN);  // (the persistent loop moves them)
  int t_last = __builtin_amdgcn_readfirstlane((kend - 1) / BN);
  // The persistent loop numbers its steps across blocks: its block starts at
  // step phase phase0 (mod 6), which sets the K (mod 2) and V (mod 3) buffer
  // of each tile, and when the next block's first two tiles follow this
  // block's last in the sequence (pf_steps), the last two steps load them
  // (nxt_first: the next block's first tile).  0, false: a single block.
  int phase0 = 0, nxt_first = 0;
  bool pf_steps = false;
  // the tile n places after tile t in this workgroup's sequence of loads
  // (past the last tile without a next block: the last tile again)
  auto ahead = [&](int t, int n) {
    if constexpr (PERS) return t + n <= t_last ? t + n : pf_steps ? nxt_first + (t + n - t_last - 1) : t_last;
    else return min(t + n, t_last);
  };

  // K/V rows of a head are kv_cap apart; logical key j is physical row
  // (ring_start + j) % kv_cap.  Without a wrap the live keys are one run of
  // rows from ring_start; with one (RING) the tile loads split at the wrap.
  const size_t kv_row = (size_t)(b * p.Hkv + hkv) * (size_t)p.kv_cap + (RING ? 0 : (size_t)p.ring_start);
  const uint16_t* __restrict__ kg = p.k + kv_row * DK;
  const uint16_t* __restrict__ vg = p.v + kv_row * DV;

  // this lane's Q row of row block mbx (zeros for a row past the block's end)
  auto load_q = [&](uint4 (&dst)[DC], int mbx) {
    const int r0 = mbx * BM, re = min(p.rows, r0 + BM);
    const int m = r0 + rb * kRowsPerWave + lr;
    const bool ok = m < re;
    const uint16_t* qrow =
        p.q + ((size_t)(b * p.Hq + hkv * p.G + (ok ? m % p.G : 0)) * p.qL + (ok ? m / p.G : 0)) * DK + qd0;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) dst[dc] = ok ? *(const uint4*)(qrow + dc * 16 + lg * 8) : make_uint4(0, 0, 0, 0);
  };
  uint4 qf[DC];
  {
    load_q(qf, mb);
    if constexpr (MT != DT) {  // bf16 Q to the fp16 of the staged tiles (RNE; exact in fp16's range)
      auto cvt = [](uint32_t w) {
        return Elem<0>::pack2(__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u));
      };
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) qf[dc] = make_uint4(cvt(qf[dc].x), cvt(qf[dc].y), cvt(qf[dc].z), cvt(qf[dc].w));
    }
  }
  // 4-bit K: the B operand of the group-constant MFMA.  Q_g, the sum of the
  // row's 64 (fp16) q elements of group g, in fp32 (the two lanes of a row
  // hold halves of each group: their sums are added in either order, a + b
  // == b + a), split into fp16 high and low parts.  Entries k = 0..15 of the
  // B column: Q_g high at k = g and 8 + g, Q_g low at k = 4 + g, zero at
  // 12..15; against the A entries b_g high at g and 4 + g and b_g low at 8 +
  // g, the product sums b_g (Q_g high + low) + b_g low Q_g high.
  // It is kept in LDS after the K operands (each lane reads back only its own
  // 16 bytes, in program order: no barrier), not in registers across the loop.
  uint16_t* const q4_qs = lds + 4 * TILE + 2 * 1024 + 8 * tid;
  auto q4_qsum = [&]() { return *(const uint4*)q4_qs; };
  if constexpr (Q4) {
    float qs[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float a = 0.f;
#pragma unroll
      for (int dc = 4 * g; dc < 4 * g + 4; ++dc) {
        const uint32_t w[4] = {qf[dc].x, qf[dc].y, qf[dc].z, qf[dc].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a += (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu)) +
               (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
      }
      qs[g] = pair_sum(a);
    }
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const _Float16 h0 = (_Float16)qs[2 * i], h1 = (_Float16)qs[2 * i + 1];
      hi[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      lo[i] = Elem<0>::pack2(qs[2 * i] - (float)h0, qs[2 * i + 1] - (float)h1);
    }
    *(uint4*)q4_qs = lg == 0 ? make_uint4(hi[0], hi[1], lo[0], lo[1]) : make_uint4(hi[0], hi[1], 0u, 0u);
  }

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float m_ref = -INFINITY;
  float l_run = 0.f;
  const float sl2 = p.sl2;

  // LDS operand offsets.  K (key row 32 kb + lr, chunk qd0 / 8 + 2 dc + lg,
  // stored at chunk position (qd0 / 8 + 2 dc + lg) ^ (lr & 15)): the swizzle
  // flips bits 3-6 of the element offset, which nothing else occupies, so
  // one per-lane base and an XOR with 16 (dc & 7) cover every dc.
  const int kbase = lr * LD + qd0 + 8 * (lg ^ (lr & 1)) + 16 * ((lr & 15) >> 1);
  auto kaddr = [&](int kb, int dc) { return (kbase ^ (16 * (dc & 7))) + 16 * (dc & 8) + kb * 32 * LD; };
  int vlane;
  {
    const int g = lane >> 4, kq = 4 * (g >> 1) + ((lane >> 2) & 3);
    vlane = kq * LD + (od0 ^ (32 * (kq & VSW))) + 16 * (g & 1) + 4 * (lane & 3);
  }
  // K(t) lives in K buffer (t - t_first) & 1, V(t) in V buffer (t - t_first)
  // & 1 (% 3 with three V buffers): the steps come in pairs (sixes), so
  // inside a step every buffer offset is a compile-time immediate of the LDS
  // instructions.  The persistent loop rotates them by its block's phase.
  uint16_t* const kbuf0 = lds;
  uint16_t* const vbuf0 = lds + 2 * TILE;
  // the K and V buffers of the block's step slots x (mod 2) and y (mod 3)
  auto kbuf_at = [&](int x) { return kbuf0 + ((x + phase0) & 1) * TILE; };
  auto vbuf_at = [&](int y) { return vbuf0 + ((y + phase0) % NVB) * TILE; };
  float* const xch = (float*)(lds + 4 * TILE);  // pair score exchange (D = 512)

  // Direct loads of one K or V tile: LOADS blocks of 1 KiB of LDS (RPB key
  // rows each) per wave, the n-th at block b = wave + NW n.  Lane l reads
  // key row l / ROWCH of the block at chunk (l % ROWCH) ^ swizzle(row) and
  // lands at LDS position l, which puts chunk c of key row r at c ^ (r & 15)
  // (K) or c ^ ((r & VSW) << 2) (V).  A lane whose chunk lies past the head
  // dim (LD > DK or DV) gets an offset outside every tile's range and writes
  // zeros.  Block b starts at key row RPB b, so the n-th load's lane offset
  // is a pattern that repeats every KPAT (K) or VPAT (V) loads plus n NW RPB
  // rows, which goes into the scalar offset.  The tile start and its bytes
  // before key kL form the buffer descriptor, so rows past kL read zeros
  // (the range check covers the scalar offset too).
  constexpr int RPB = 1024 / (2 * LD);  // key rows per 1 KiB block
  // the n-th load of this wave fills block blk(n): wave + NW n, or with GRP
  // LOADS wave + n; its lane offsets repeat every KPAT (K) or VPAT (V) loads
  constexpr int KPAT = GRP ? (16 / RPB < LOADS ? 16 / RPB : LOADS) : 16 / (NW * RPB) > 1 ? 16 / (NW * RPB) : 1;
  constexpr int VPAT = GRP ? ((VSW + 1) / RPB < LOADS ? (VSW + 1) / RPB : LOADS)
                           : (VSW + 1) / (NW * RPB) > 1 ? (VSW + 1) / (NW * RPB) : 1;
  auto blk = [&](int n) { return GRP ? LOADS * wave + n : wave + NW * n; };
  static_assert(RPB * ROWCH == 64 && LOADS % KPAT == 0 && LOADS % VPAT == 0, "block geometry");
  // above any tile's bytes, and far enough below 2^32 that adding a scalar
  // offset cannot wrap it
  constexpr uint32_t kPastRange = 0x40000000u;
  auto row_bytes = [](bool is_v) { return 2 * (is_v ? DV : DK); };
  auto lane_off = [&](bool is_v, int n) {  // offset of the n-th load from its block group
    const int r = blk(n) * RPB + lane / ROWCH;  // key row in the tile
    const int pch = lane % ROWCH;
    const int c = is_v ? (pch ^ ((r & VSW) << 2)) : (pch ^ (r & 15));
    const int rn = GRP ? n * RPB : n * NW * RPB;  // rows the scalar and immediate offsets hold
    return 16 * c < row_bytes(is_v) ? (uint32_t)((r - rn) * row_bytes(is_v) + 16 * c) : kPastRange;
  };
  uint32_t koff[KPAT], voff[VPAT];
#pragma unroll
  for (int i = 0; i < KPAT; ++i) koff[i] = lane_off(false, i);
#pragma unroll
  for (int i = 0; i < VPAT; ++i) voff[i] = lane_off(true, i);
  // A tile's source.  Without RING: one descriptor from the tile's first
  // row.  With RING the tile's rows r < r0 are physical rows bp + r (bp the
  // physical row of its first key) and rows r >= r0 wrap to physical r - r0:
  // descriptor a from row bp, descriptor b from r0 rows before the head's
  // first row (only lanes with r >= r0 read through it).
  struct TileSrc {
    i32x4_t a, b;
    int r0;  // rows of the tile before the ring wraps (BN: none)
  };
  auto tile_src = [&](const uint16_t* g, int t, bool is_v) {
    const int rowb = row_bytes(is_v);
    const int ts = __builtin_amdgcn_readfirstlane(t * BN);
    const int bytes = __builtin_amdgcn_readfirstlane(min(p.kL - ts, BN) * rowb);
    TileSrc src;
    if constexpr (!RING) {
      src.a = tile_rsrc(uniform_addr(g + (size_t)ts * (rowb / 2)), bytes);
      src.b = src.a;
      src.r0 = BN;
    } else {
      int bp = p.ring_start + ts;  // < 2 kv_cap: ring_start < kv_cap, ts < kL <= kv_cap
      if (bp >= p.kv_cap) bp -= p.kv_cap;
      bp = __builtin_amdgcn_readfirstlane(bp);
      const int r0 = __builtin_amdgcn_readfirstlane(min(p.kv_cap - bp, BN));
      const uint64_t head = uniform_addr(g);
      src.a = tile_rsrc(head + (uint64_t)bp * rowb, min(r0 * rowb, bytes));
      src.b = tile_rsrc(head - (uint64_t)r0 * rowb, bytes);
      src.r0 = r0;
    }
    return src;
  };
  auto load_blk = [&](const TileSrc& src, uint16_t* buf, int n, bool is_v) {
    if constexpr (Q4) return;  // 4-bit tiles come through registers (below)
    const uint32_t vo = is_v ? voff[n % VPAT] : koff[n % KPAT];
    uint16_t* dst = buf + blk(n) * 512;
    if constexpr (GRP) {
      // group n / 4 of this wave's blocks: scalar offset and M0 at its first
      // block, load n % 4 of the group through the immediate offset
      const uint32_t so = (uint32_t)((n & ~3) * 1024);
      const unsigned mb = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(buf + LOADS * wave * 512));
      const unsigned mo = (unsigned)((n & ~3) * 1024);
      switch (n & 3) {
        case 0: load_lds16_grp<0>(src.a, vo, so, mb, mo); break;
        case 1: load_lds16_grp<1>(src.a, vo, so, mb, mo); break;
        case 2: load_lds16_grp<2>(src.a, vo, so, mb, mo); break;
        default: load_lds16_grp<3>(src.a, vo, so, mb, mo); break;
      }
      return;
    }
    const uint32_t so = (uint32_t)(n * NW * RPB * row_bytes(is_v));
    if constexpr (PERS) {  // its buffers rotate with the block's phase: one base each
      load_lds16_off(src.a, vo, so, __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(buf + wave * 512)),
                     (unsigned)(NW * n * 1024));
    } else if constexpr (!RING) {
      load_lds16(src.a, vo, so, dst);
    } else {
      // lanes of rows before the wrap: lanes [LPR i, LPR (i + 1)) hold row
      // i of the block's RPB rows
      constexpr int LPR = 64 / RPB;
      const int rb0 = blk(n) * RPB;
      uint64_t ea = 0;
#pragma unroll
      for (int i = 0; i < RPB; ++i)
        if (rb0 + i < src.r0) ea |= (LPR == 64 ? ~0ull : ((1ull << LPR) - 1ull) << (LPR * i));
      load_lds16_2(src.a, src.b, uniform64(ea), uniform64(~ea), vo, so,
                   __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst));
    }
  };
  auto load_tile = [&](const uint16_t* g, int t, uint16_t* buf, bool is_v) {
    const TileSrc src = tile_src(g, t, is_v);
    const unsigned m0 = m0_save();
#pragma unroll
    for (int n = 0; n < LOADS; ++n) load_blk(src, buf, n, is_v);
    m0_restore(m0);
  };
  auto load_k = [&](int t) { load_tile(kg, t, kbuf0 + ((t - t_first + phase0) & 1) * TILE, false); };

  // Additive mask array (BIAS).  A bias tile holds this workgroup's BM
  // packed rows x BN keys for one K/V tile, in LDS after K, V (and the pair
  // exchange), double-buffered like K: bias(t) is in bias buffer
  // (t - t_first) & 1 and is loaded with K(t).  Chunk c (8 keys) of tile row
  // r sits at chunk position c ^ (r & (BCPR - 1)), so the 32 rows a read
  // touches spread over the banks.  A lane's load offsets are loop-invariant
  // (its row's (query head, position) and its chunk); rows past the
  // workgroup's last row point out of the descriptor's range and read zeros,
  // keys past kL read the next row's entries, whose scores are masked.
  constexpr int BTILE = BM * BN, BCPR = BN * 2 / 16, BRPB = 64 / BCPR;
  constexpr int BLOADS = BIAS ? BTILE * 2 / 1024 / NW : 0;
  static_assert(!BIAS || (BLOADS >= 1 && BRPB * BCPR == 64 && !RING), "bias tile geometry");
  uint16_t* const bbuf0 = lds + 4 * TILE + (PAIR ? 2 * 4 * 64 * 16 : 0);
  uint32_t boff[BLOADS > 0 ? BLOADS : 1];
  int bbase = 0;
  int64_t bias_extent = 0;
  const uint16_t* bias_b = nullptr;
  // The descriptor's range ends exactly at the end of batch b's bias extent
  // (bias_src below), and its range check is per 4-byte word; a row's words
  // start at its first element.  So with kL odd, the word that holds key
  // kL - 1 of a row that ends the extent also covers the 2 bytes after the
  // extent: it is out of range and reads as zero, and nothing past the
  // extent is read.  That one element is written into the tile afterwards
  // (bias_patch): a lane whose load n covers it has bit n of bpatch set,
  // bias_last is its value (one 2-byte load from inside the extent) and
  // bpatch_e its place in the lane's 8 elements.  Only the tile holding key
  // kL - 1 (t_bend) needs it.
  uint32_t bpatch = 0;
  uint32_t bias_last = 0;
  int bpatch_e = 0;
  const int t_bend = __builtin_amdgcn_readfirstlane((p.kL - 1) / BN);
  if constexpr (BIAS) {
    bias_b = p.bias + b * p.bias_sb;
    bias_extent = (int64_t)(p.Hq - 1) * p.bias_sh + (int64_t)(p.qL - 1) * p.bias_sq + p.kL;
    const int64_t last_row = bias_extent - p.kL;         // start of the rows that end the extent
    const int c_last = ((p.kL - 1) % BN) / 8;             // chunk of key kL - 1 within its tile
    bpatch_e = (p.kL - 1) % 8;
#pragma unroll
    for (int n = 0; n < BLOADS; ++n) {
      const int r = (wave + NW * n) * BRPB + lane / BCPR;  // bias tile row
      const int c = (lane % BCPR) ^ (r & (BCPR - 1));
      const int prow = row0 + r;
      const int pq = prow / p.G, ph = hkv * p.G + prow % p.G;
      const int64_t start = (int64_t)ph * p.bias_sh + (int64_t)pq * p.bias_sq;
      boff[n] = prow < rows_end ? (uint32_t)((start + 8 * c) * 2) : 0xfffffff0u;
      if ((p.kL & 1) && prow < rows_end && start == last_row && c == c_last) bpatch |= 1u << n;
    }
    if ((p.kL & 1) && t_last == t_bend) bias_last = bias_b[bias_extent - 1];
    else bpatch = 0;
    const int r = rb * kRowsPerWave + lr;  // this lane's row in the bias tile
    bbase = r * BN + 8 * (r & (BCPR - 1)) + 4 * lg;
  }
  // batch b's bias from key t BN to the end of its extent
  auto bias_src = [&](int t) {
    const int ts = __builtin_amdgcn_readfirstlane(t * BN);
    return tile_rsrc(uniform_addr(bias_b + ts),
                     __builtin_amdgcn_readfirstlane((int)(uint32_t)((bias_extent - ts) * 2)));
  };
  // after this wave's loads of tile t into bias buffer buf have landed and
  // before the barrier that publishes it: the element the range check zeroed
  auto bias_patch = [&](int t, uint16_t* buf) {
    if constexpr (BIAS) {
      if (t == t_bend && bpatch != 0) {
#pragma unroll
        for (int n = 0; n < BLOADS; ++n)
          if (bpatch & (1u << n)) buf[(wave + NW * n) * 512 + 8 * lane + bpatch_e] = (uint16_t)bias_last;
      }
    }
  };
  auto load_bblk = [&](const i32x4_t& src, uint16_t* buf, int n) {
    load_lds16(src, boff[n], 0u, buf + (wave + NW * n) * 512);
  };
  auto load_b = [&](int t) {
    if constexpr (BIAS) {
      const i32x4_t src = bias_src(t);
      const unsigned m0 = m0_save();
#pragma unroll
      for (int n = 0; n < BLOADS; ++n) load_bblk(src, bbuf0 + ((t - t_first) & 1) * BTILE, n);
      m0_restore(m0);
    }
  };
  // the 4-key groups of bias a lane needs for one tile (group g holds the
  // keys of score elements 4 g .. 4 g + 3), and one element's value in the
  // units of the raw q.k scores the kernel keeps (bias / scale: the softmax
  // takes exp2(s scale log2 e), so s + bias / scale gives scale s + bias)
  const float inv_scale = p.inv_scale;
  auto bias_read = [&](const uint16_t* bl, int g) { return *(const uint2*)(bl + (bbase ^ (8 * g))); };
  auto bias_val = [&](const uint2 (&bw)[KB * 4], int e) {
    const uint32_t w = (e % 4) < 2 ? bw[e / 4].x : bw[e / 4].y;
    const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xffffu);
    float x;
    if constexpr (DT == 1) x = __builtin_bit_cast(float, h << 16);
    else x = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    return x * inv_scale;
  };
  auto load_v = [&](int t) { load_tile(vg, t, vbuf0 + ((t - t_first + phase0) % NVB) * TILE, true); };

  // ---- 4-bit K/V (Q4) ------------------------------------------------------
  // A 1 KiB LDS block of a tile gets, per lane, the 8 elements the direct
  // load would have written there (key row r of the block's RPB rows, chunk
  // c after the K or V swizzle): one 32-bit code word, the scale and the
  // bias of its 64-element group, then fp32 scale * code + bias for each
  // nibble, rounded to the input dtype.  The rows are those of a KV cache
  // (kv_cap rows per head, logical key j in row (ring_start + j) mod
  // kv_cap), wrapped per lane.  Rows past kL repeat row kL - 1
  // (finite values; their keys are masked, so their weights are exactly 0):
  // no branch around a load, so the loads' waits stay counted.
  // Loading waves: with one row-holding wave (G * qL <= 32 rows in the
  // workgroup, a decode or verify step) the other three load, one step
  // ahead through two register sets (q4 pipelined), and the computing wave
  // issues no loads; otherwise every wave loads its share, issued at the
  // start of a step and written to LDS at its end.
  constexpr int NBLK = TILE * 2 / 1024;   // 1 KiB blocks per tile
  constexpr int QB = (NBLK + 2) / 3;      // blocks per tile per loader of three (decode)
  constexpr int QB4 = NBLK / 4;           // blocks per tile per wave when all four load
  struct Q4Data {  // loaded values only: nothing is computed from them before the store
    uint32_t w;     // code word
    uint32_t s, b;  // scale and bias bit patterns
  };
  // waves 1..3 load, one step ahead (always in the decode instance; in the
  // general one when the workgroup has a single row-holding wave)
  const int n_act = __builtin_amdgcn_readfirstlane(min(NW, (rows_end - row0 + kRowsPerWave - 1) / kRowsPerWave));
  const bool q4_pipe = Q4M == 1 || (Q4M == 2 && n_act == 1);
  const int q4_nl = q4_pipe ? NW - 1 : NW;        // loading waves
  const int q4_li = q4_pipe ? wave - 1 : wave;    // this wave's index among them
  const size_t q4_head = (size_t)(b * p.Hkv + hkv) * (size_t)p.kv_cap;  // the head's first cache row
  const uint32_t* const q4_kq = p.kq4 + q4_head * (DK / 8);
  const uint32_t* const q4_vq = p.vq4 + q4_head * (DK / 8);
  const uint16_t* const q4_ks = p.ks4 + q4_head * (DK / 64);
  const uint16_t* const q4_kb = p.kb4 + q4_head * (DK / 64);
  const uint16_t* const q4_vs = p.vs4 + q4_head * (DK / 64);
  const uint16_t* const q4_vb = p.vb4 + q4_head * (DK / 64);
  auto q4_fetch = [&](int t, int blk, bool is_v) {
    const int r = blk * RPB + lane / ROWCH, pch = lane % ROWCH;
    const int c = is_v ? (pch ^ ((r & VSW) << 2)) : (pch ^ (r & 15));
    const int key = min(t * BN + r, p.kL - 1);
    // logical key -> cache row: (ring_start + key) mod kv_cap, by one select
    // (ring_start < kv_cap and key < kL <= kv_cap)
    int phys = p.ring_start + key;
    phys = phys >= p.kv_cap ? phys - p.kv_cap : phys;
    Q4Data d{0u, 0u, 0u};
    if constexpr (Q4) {
      // 32-bit byte offsets from the head's first row (a head's code words
      // stay below 4 GiB: the entry point bounds kv_cap)
      const uint32_t wb = ((uint32_t)phys * (DK / 8) + (uint32_t)c) * 4u;
      const uint32_t gb = ((uint32_t)phys * (DK / 64) + (uint32_t)(c / 8)) * 2u;
      d.w = *(const uint32_t*)((const char*)(is_v ? q4_vq : q4_kq) + wb);
      d.s = *(const uint16_t*)((const char*)(is_v ? q4_vs : q4_ks) + gb);
      d.b = *(const uint16_t*)((const char*)(is_v ? q4_vb : q4_kb) + gb);
    }
    return d;
  };
  auto q4_widen = [](uint32_t h) {
    if constexpr (DT == 1) return __builtin_bit_cast(float, h << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  };
  // K(t)'s group-constant operand: per key row r of the tile, 16 fp16 entries
  // at q4_kc + ((t - t_first) & 1) * 1024 + 16 r (see the K elements below)
  uint16_t* const q4_kc = lds + 4 * TILE;
  auto q4_store = [&](const Q4Data& d, uint16_t* buf, int blk, bool is_k) {
    const float sc = q4_widen(d.s);
    // V: element scale * code + bias.  K: the centred element scale *
    // (code - 8), exact in fp16 for a bf16 scale (8 significant bits times an
    // integer of at most 3), and the group's constant bias + 8 scale goes to
    // the key row's operand entries g, g + 4 (its fp16 high part) and 8 + g
    // (the low part), written by the lane holding the group's first chunk;
    // the scores take it through one MFMA per key block against the
    // query's group sums (q4_qsum)
    const float bi = is_k ? -8.f * sc : q4_widen(d.b);
    if (is_k) {
      const int r = blk * RPB + lane / ROWCH, c = (lane % ROWCH) ^ (r & 15);
      if ((c & 7) == 0) {
        const float bg = q4_widen(d.b) + 8.f * sc;
        const _Float16 h = (_Float16)bg;
        const _Float16 l = (_Float16)(bg - (float)h);
        uint16_t* e = q4_kc + (buf == kbuf0 ? 0 : 1024) + 16 * r + c / 8;
        e[0] = __builtin_bit_cast(uint16_t, h);
        e[4] = __builtin_bit_cast(uint16_t, h);
        e[8] = __builtin_bit_cast(uint16_t, l);
      }
    }
    // even elements' codes in the bytes of lo, odd ones' in the bytes of hi:
    // each code is then one byte-to-float conversion (v_cvt_f32_ubyte<k>).
    // The empty asm hides that the bytes' high nibbles are zero; knowing it,
    // the compiler forms a bit-field extract and a byte-0 conversion per
    // code instead, twice the instructions
    uint32_t lo = d.w & 0x0F0F0F0Fu, hi = (d.w >> 4) & 0x0F0F0F0Fu;
    asm("" : "+v"(lo), "+v"(hi));
    auto val = [&](uint32_t x, auto kc) {
      constexpr int k = decltype(kc)::value;
      return fmaf(sc, (float)((x >> (8 * k)) & 0xFFu), bi);
    };
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    using K3 = std::integral_constant<int, 3>;
    uint4 out;
    out.x = EM::pack2(val(lo, K0{}), val(hi, K0{}));
    out.y = EM::pack2(val(lo, K1{}), val(hi, K1{}));
    out.z = EM::pack2(val(lo, K2{}), val(hi, K2{}));
    out.w = EM::pack2(val(lo, K3{}), val(hi, K3{}));
    *(uint4*)(buf + blk * 512 + 8 * lane) = out;
  };
  // this wave's blocks of K tile tk and V tile tv: issue, then store.
  // Slots past the last block repeat it (the same bytes written twice), so
  // that no branch separates a load from its store and every wait counts
  auto q4_blk = [&](int i) { return min(q4_li + q4_nl * i, NBLK - 1); };
  auto q4_issue = [&](auto& kd, auto& vd, int tk, int tv) {
    constexpr int N = sizeof(kd) / sizeof(kd[0]);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      kd[i] = q4_fetch(tk, q4_blk(i), false);
      vd[i] = q4_fetch(tv, q4_blk(i), true);
    }
  };
  auto q4_put = [&](const auto& kd, const auto& vd, uint16_t* kdst, uint16_t* vdst) {
    constexpr int N = sizeof(kd) / sizeof(kd[0]);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      q4_store(kd[i], kdst, q4_blk(i), true);
      q4_store(vd[i], vdst, q4_blk(i), false);
    }
  };

  // the keys row `pos` sees form one interval [key_lo, key_hi] (empty if
  // key_hi < key_lo)
  int key_lo, key_hi;
  auto set_keys = [&]() {
    key_lo = p.window > 0 ? max(0, pos - p.window + 1) : 0;
    key_hi = p.causal ? min(pos, p.kL - 1) : p.kL - 1;
  };
  set_keys();
  auto full_tile = [&](int t) {  // every key of tile t visible to every row of this wave
    const int ts = t * BN, te = ts + BN - 1;
    return (te < p.kL) && (!p.causal || te <= wp_lo) && (p.window == 0 || ts >= wp_hi - p.window + 1);
  };

  // ---- building blocks (inlined; no scheduling barriers, so that callers
  //      can interleave them with sched_group_barrier patterns) -------------
  // S^T = K(t) Q^T, K operands read PF MFMAs ahead; the two key-block chains
  // alternate
  // 4-bit K: the A operand of the group-constant MFMA of key block kb, from
  // the operand entries of the K buffer whose tile starts at kl
  auto q4_kc_read = [&](const uint16_t* kl, int kb) {
    return *(const uint4*)(q4_kc + (kl == kbuf0 ? 0 : 1024) + 16 * (32 * kb + lr) + 8 * lg);
  };
  auto qk = [&](f32x16_t (&s)[KB], const uint16_t* kl) {
    constexpr int PF = 4;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
    if constexpr (Q4) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = EM::mfma(q4_kc_read(kl, kb), q4_qsum(), s[kb]);
    }
    auto kread = [&](int n) {
      const int kb = n % KB, dc = n / KB;
      return *(const uint4*)(kl + kaddr(kb, dc));
    };
    uint4 a[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) a[i] = kread(i);
#pragma unroll
    for (int n = 0; n < NQK; ++n) {
      const uint4 cur_a = a[n % PF];
      if (n + PF < NQK) a[n % PF] = kread(n + PF);
      s[n % KB] = EM::mfma(cur_a, qf[n / KB], s[n % KB]);
    }
  };
  // keys of tile t a row may not see -> -inf.  Score element (kb, j) holds
  // key ts + 4 lg + c with c = 32 kb + 8 (j / 4) + j % 4 a compile-time
  // constant, so it is visible iff lo4 <= c <= hi4 for two per-tile values:
  // the tile's visibility is a 64-bit mask over c, and each element takes a
  // bit extract and a bit-field insert of -inf.  Only tiles that are not
  // wholly visible to the wave's rows come here (a uniform branch).
  auto mask = [&](f32x16_t (&s)[KB], int t) {
    const int lo4 = key_lo - t * BN - 4 * lg, hi4 = key_hi - t * BN - 4 * lg;
    const int lo = min(max(lo4, 0), 64), hi = min(max(hi4 + 1, 0), 64);  // visible c in [lo, hi)
    auto ones = [](int n) { return n >= 32 ? 0xffffffffu : ((1u << n) - 1u); };  // n in [0, 32]
    const uint32_t vmask[2] = {ones(min(hi, 32)) & ~ones(min(lo, 32)), ones(max(hi - 32, 0)) & ~ones(max(lo - 32, 0))};
    const uint32_t ninf_bits = __builtin_amdgcn_readfirstlane(0xff800000u);  // -inf, in an SGPR
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c = 32 * kb + 8 * (j >> 2) + (j & 3);
        s[kb][j] = bit_select(__builtin_amdgcn_sbfe((int)vmask[c / 32], c % 32, 1), s[kb][j], ninf_bits);
      }
  };
  // row max of S(t) -> reference update; returns the factor the running
  // output and sum take before tile t is added
  auto row_max = [&](f32x16_t (&s)[KB]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
    mx = pair_max(mx);
    const bool upd = mx * sl2 > m_ref * sl2 + kRescaleLog2;
    const float alpha = upd ? ((m_ref == -INFINITY) ? 0.f : fast_exp2((m_ref - mx) * sl2)) : 1.f;
    m_ref = upd ? mx : m_ref;
    return alpha;
  };
  auto rescale = [&](float alpha) {  // x * 1 == x: most tiles skip it
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
    }
  };

  // K operand of S MFMA n: key block n % KB, d step n / KB; the XOR part of
  // its address is a register, the rest an immediate
  auto kx = [&](int n) { return kbase ^ (16 * ((n / KB) & 7)); };
  auto kread_at = [&](const uint16_t* kl, int n, int x) {
    return *(const uint4*)(kl + x + 16 * ((n / KB) & 8) + (n % KB) * 32 * LD);
  };
  // V^T operand of P V MFMA n: key half n / DB, column block n % DB; the
  // XOR part of the address is a register, the rest an immediate
  auto vx = [&](int n) { return vlane ^ (32 * (n % DB)); };
  auto vread_at = [&](const uint16_t* vl, int n, int x) {
    const uint16_t* va = vl + x + 16 * (n / DB) * LD;
    const uint2 lo = read_tr(va), hi = read_tr(va + 8 * LD);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };

  // ---- interleaved regions: slot n issues MFMA n, the operand read for MFMA
  //      n + PF and a share of the other tile's vector work; the scheduling
  //      barriers keep that order.  With one wave per SIMD, instructions
  //      issue in order, so a vector op that needs the result of the op just
  //      before it stalls the MFMA stream: every dependency chain (address ->
  //      LDS read, fma -> exp -> sum, compare -> select -> max) is spread
  //      over consecutive slots instead.
  // S(t+1) = K(t+1) Q^T  ||  weights, sum and packing of tile t; also issues
  // the direct loads of K(tk) (and its bias tile) into kdst (bdst), and
  // unless VLATE those of V(tv) into vdst
  auto qk_weights = [&](f32x16_t (&sn)[KB], const uint16_t* kl, f32x16_t (&sc)[KB],
                        uint4 (&pb)[KB * 2], const TileSrc& ksrc, uint16_t* kdst, const TileSrc& vsrc,
                        uint16_t* vdst, const i32x4_t& bsrc, uint16_t* bdst, const uint16_t* bl,
                        uint2 (&bw)[KB * 4], uint4 (&a)[4], const uint4 (&kc)[KB + 1]) {
    constexpr int PF = 4;
    // the slots of K block group i, V block group i (unless VLATE) and bias
    // block group i: spread evenly over the region, V half a spacing after
    // K, bias one slot after K (two when runs are three slots long, so as
    // not to share V's).  When the slots divide evenly the tests are written
    // as runs of LS slots (the form the compiler schedules best); otherwise
    // slot by slot.
    static_assert(NQK >= 2 * LOADS, "slot pattern");
    constexpr bool EVEN = NQK % LOADS == 0;
    constexpr int LS = NQK / LOADS, BSLOT = LS == 3 ? 2 : 1;
    auto kslot = [](int i) { return i * NQK / LOADS; };
    auto vslot = [](int i) { return (2 * i + 1) * NQK / (2 * LOADS); };
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sn[kb][j] = 0.f;
    if constexpr (Q4) {  // the key rows' group constants times the query's group sums first
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sn[kb] = EM::mfma(kc[kb], kc[KB], sn[kb]);
    }
    // K operand of MFMA n: key block n % KB, d step n / KB; the XOR part of
    // its address is a register, the rest an immediate
    auto kread = [&](int n, int x) { return kread_at(kl, n, x); };
    const float msc = (m_ref == -INFINITY) ? 0.f : m_ref * sl2;
    auto get = [&](int e) { return sc[e / 16][e % 16]; };
    auto set = [&](int e, float v) { sc[e / 16][e % 16] = v; };
    float psum = 0.f;
    int x_next = kx(PF);
    const unsigned m0 = m0_save();
    // weights in slot n: fma of the elements of slot n + 2, exp of those of
    // slot n + 1, sum and pack of its own (elements [es(m), es(m + 1)) are
    // slot m's)
#pragma unroll
    for (int e = es(0); e < es(1); ++e) set(e, fast_exp2(get(e) * sl2 - msc));
#pragma unroll
    for (int e = es(1); e < es(2); ++e) set(e, get(e) * sl2 - msc);
    // the pairs slot m packs: its odd elements e, pair (e - 1, e); at most two
    auto npacks = [&](int m) {
      int c = 0;
      for (int e = es(m); e < es(m + 1); ++e) c += e & 1;
      return c;
    };
    uint32_t wlast[2] = {0, 0};  // the words the last slot packed
#pragma unroll
    for (int n = 0; n < NQK; ++n) {
      const uint4 cur_a = a[n % PF];
      if (n + PF < NQK) a[n % PF] = kread(n + PF, x_next);
      sn[n % KB] = EM::mfma(cur_a, qf[n / KB], sn[n % KB]);
      if (n + PF + 1 < NQK) x_next = kx(n + PF + 1);
      // loads: K, V and bias block group i at slots kslot(i), vslot(i), bslot(i)
      if constexpr (EVEN) {
        if (n % LS == 0) load_blk(ksrc, kdst, n / LS, false);
        if (!VLATE && n % LS == LS / 2) load_blk(vsrc, vdst, n / LS, true);
      } else {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          if (n == kslot(i)) load_blk(ksrc, kdst, i, false);
          if (!VLATE && n == vslot(i)) load_blk(vsrc, vdst, i, true);
        }
      }
      if constexpr (BIAS) {
        // the bias tile that goes with K(tk), and in the last slots the bias
        // of S(t + 1) for the P V region (its reads are in flight by then)
        if constexpr (EVEN) {
          if (n % LS == BSLOT && n / LS < BLOADS) load_bblk(bsrc, bdst, n / LS);
        } else {
#pragma unroll
          for (int i = 0; i < BLOADS; ++i)
            if (n == kslot(i) + 1) load_bblk(bsrc, bdst, i);
        }
        if (n >= NQK - KB * 4) bw[n - (NQK - KB * 4)] = bias_read(bl, n - (NQK - KB * 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ef = es(n + 2) + i, ex = es(n + 1) + i;
        if (ef < es(n + 3)) set(ef, get(ef) * sl2 - msc);
        if (ex < es(n + 2)) set(ex, fast_exp2(get(ex)));
      }
      // the row sum adds the rounded weights the P V product uses, a pair
      // per dot2, one slot after the pair is packed
      if (n > 0) {
#pragma unroll
        for (int i = 0; i < npacks(n - 1); ++i) psum = EM::sum2(wlast[i], psum);
      }
#pragma unroll
      for (int e = es(n); e < es(n + 1); ++e) {
        if (e & 1) {  // pack the pair (e - 1, e): P half kh = e / 8
          const uint32_t w = EM::pack2(get(e - 1), get(e));
          wlast[e - es(n) > 1 ? 1 : 0] = w;
          uint4& q = pb[e / 8];
          switch ((e % 8) / 2) {
            case 0: q.x = w; break;
            case 1: q.y = w; break;
            case 2: q.z = w; break;
            default: q.w = w; break;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < npacks(NQK - 1); ++i) psum = EM::sum2(wlast[i], psum);
    m0_restore(m0);
    // an empty volatile use: the sum is formed here, slot by slot, not sunk
    // past the next region as a serial chain
    asm volatile("" ::"v"(psum));
    return psum;
  };
  // O += P(t) V(t)  ||  row max of S(t+1) (already masked); with VLATE also
  // issues the direct loads of V(tv) into vdst, one block group every LSV
  // slots
  auto pv_max = [&](const uint4 (&pb)[KB * 2], const uint16_t* vl, f32x16_t (&sn)[KB], bool live,
                    const uint2 (&bw)[KB * 4], const TileSrc& vsrc, uint16_t* vdst) {
    constexpr int PF = 4;
    static_assert(NPV % LOADS == 0 && NPV >= LOADS, "V load slot pattern");
    constexpr int LSV = NPV / LOADS;
    // V^T operand of MFMA n: key half n / DB, column block n % DB; the XOR
    // part of the address is a register, the rest an immediate
    auto vread = [&](int n, int x) { return vread_at(vl, n, x); };
    auto get = [&](int e) { return sn[e / 16][e % 16]; };
    float mx = -INFINITY;
    // BIAS: the elements a slot's max takes get their bias one slot before
    auto add_bias = [&](int slot) {
      if constexpr (BIAS) {
#pragma unroll
        for (int e = ev(slot); e < ev(slot + 1); ++e) sn[e / 16][e % 16] = get(e) + bias_val(bw, e);
      }
    };
    add_bias(0);
    uint4 bv[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) bv[i] = vread(i, vx(i));
    int x_next = vx(PF);
    const unsigned m0 = VLATE ? m0_save() : 0u;
#pragma unroll
    for (int n = 0; n < NPV; ++n) {
      const uint4 cur_b = bv[n % PF];
      if (n + PF < NPV) bv[n % PF] = vread(n + PF, x_next);
      o[n % DB] = EM::mfma(cur_b, pb[n / DB], o[n % DB]);
      if (n + PF + 1 < NPV) x_next = vx(n + PF + 1);
      if (VLATE && n % LSV == LSV / 2) load_blk(vsrc, vdst, n / LSV, true);
      // the pairs (e - 1, e) whose odd element is one of this slot's
#pragma unroll
      for (int e = ev(n); e < ev(n + 1); ++e)
        if (e & 1) mx = max3(mx, get(e - 1), get(e));
      add_bias(n + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (VLATE) m0_restore(m0);
    mx = pair_max(mx);
    // live == false: the scores were of no tile (the step after the last)
    const bool upd = live && (mx * sl2 > m_ref * sl2 + kRescaleLog2);
    const float alpha = upd ? ((m_ref == -INFINITY) ? 0.f : fast_exp2((m_ref - mx) * sl2)) : 1.f;
    m_ref = upd ? mx : m_ref;
    return alpha;
  };

  // Direct loads a VLATE step issues in its S region (K(t+2) and its bias
  // tile) and in its P V region (V(t+1)); a wrapped ring issues two loads
  // per block
  constexpr int S_LOADS = LOADS * (RING ? 2 : 1) + BLOADS, PV_LOADS = LOADS * (RING ? 2 : 1);

  // D = 512: complete this wave's partial scores with the partner's (every
  // wave of the workgroup passes the barrier; waves without rows only wait).
  // The barrier also publishes V(t): each wave first waits for its own V(t)
  // loads, the ones it issued before its S region's loads.
  auto exchange = [&](f32x16_t (&s)[KB], bool active) {
    if constexpr (PAIR) {
      if (active) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(float4*)(xch + (wave * 4 + q4) * 256 + lane * 4) =
              make_float4(s[0][4 * q4 + 0], s[0][4 * q4 + 1], s[0][4 * q4 + 2], s[0][4 * q4 + 3]);
      }
      wait_vmem<S_LOADS>();
      __syncthreads();
      if (active) {
        const float* px = xch + (wave ^ 1) * 4 * 256 + lane * 4;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 x = *(const float4*)(px + q4 * 256);
          s[0][4 * q4 + 0] += x.x;
          s[0][4 * q4 + 1] += x.y;
          s[0][4 * q4 + 2] += x.z;
          s[0][4 * q4 + 3] += x.w;
        }
      }
    }
  };

  // ---- one row block: prologue and step loop ---------------------------
  // pf (persistent loop): 0, nothing loaded yet; 1, the block's Q rows and
  // K(t0), V(t0), K(t0 + 1) were loaded while the previous block's output
  // was stored; 2, the Q rows so, and K and V of t0 and t0 + 1 by the
  // previous block's last two steps.
  auto run_block = [&](int pf) {
    // ---- prologue: K(t0), V(t0), K(t0 + 1); S(t0) and its row max ------------
    // Rows past kL are out of the loads' range.  When this workgroup's last
    // tile has such rows, the V buffers start as zeros, so that those rows of
    // a V tile never hold uninitialised LDS (a zero weight times a NaN bit
    // pattern would still be NaN); K rows past kL need nothing, their scores
    // are masked to -inf.  (The persistent loop zeroes them once, before its
    // first block: rows past kL are never loaded, and a later block finds
    // there what an earlier tile or the zeroing left, finite either way.)
    if constexpr (Q4) {  // operand entries 12..15 of the 2 x 64 key rows: zero, never written again
      if (tid < 2 * BN) *(uint2*)(q4_kc + 16 * tid + 12) = make_uint2(0, 0);
    }
    if (!PERS && (t_last + 1) * BN > p.kL) {
      uint4* vz = (uint4*)vbuf0;
      for (int i = tid; i < NVB * TILE / 8; i += NW * 64) vz[i] = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }
    // Q4: the pipelined loaders' first register set, K(t0 + 2) and V(t0 + 1)
    // With every wave loading, two sets of this wave's QB4 blocks: set P
    // holds K(t+2), V(t+1) when step t (parity P) starts, issued one step
    // earlier; the step issues the other set for K(t+3), V(t+2)
    typename std::conditional<Q4, Q4Data, char>::type q4a_k[Q4 ? QB : 1], q4a_v[Q4 ? QB : 1];
    typename std::conditional<Q4, Q4Data, char>::type q4s_k[2][Q4M == 2 ? QB4 : 1], q4s_v[2][Q4M == 2 ? QB4 : 1];
    if constexpr (Q4) {
      if (q4_li >= 0) {  // wave 0 of a pipelined workgroup does not load
        Q4Data k0[QB], v0[QB], k1[QB], v1[QB];
        q4_issue(k0, v0, t_first, t_first);
        q4_issue(k1, v1, min(t_first + 1, t_last), t_first);
        q4_put(k0, v0, kbuf0, vbuf0);
        q4_put(k1, v1, kbuf0 + TILE, vbuf0);  // V(t0) again, the same bytes
        if (q4_pipe) q4_issue(q4a_k, q4a_v, min(t_first + 2, t_last), min(t_first + 1, t_last));
        else q4_issue(q4s_k[0], q4s_v[0], min(t_first + 2, t_last), min(t_first + 1, t_last));
      }
    } else {
      if (pf == 0) {
        load_k(t_first);
        load_b(t_first);
        load_v(t_first);
        if (t_first < t_last) {
          load_k(t_first + 1);
          load_b(t_first + 1);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      bias_patch(t_first, bbuf0);
      if (t_first < t_last) bias_patch(t_first + 1, bbuf0 + BTILE);
    }
    __syncthreads();
    // V3: V(t0 + 1) is first read in step t0 + 1, so it loads now, in flight
    // through S(t0) and step t0, whose closing wait (everything but that
    // step's own V loads) and barrier publish it
    if constexpr (V3)
      if (pf != 2 && t_first < t_last) load_v(t_first + 1);

    f32x16_t sA[KB], sB[KB];
    float alpha_cur = 1.f;
    if (wave_active) qk(sA, kbuf_at(0));
    exchange(sA, wave_active);
    if (wave_active) {
      if constexpr (BIAS) {
        uint2 bw0[KB * 4];
#pragma unroll
        for (int g = 0; g < KB * 4; ++g) bw0[g] = bias_read(bbuf0, g);
#pragma unroll
        for (int e = 0; e < NE; ++e) sA[e / 16][e % 16] += bias_val(bw0, e);
      }
      if (!full_tile(t_first)) mask(sA, t_first);
      alpha_cur = row_max(sA);
    }
    __syncthreads();  // every wave is done with K(t0) before K(t0 + 2) overwrites it

    // One pipelined step: tile t's scores are in sc, tile t + 1's go to sn.
    // Straight-line for every tile: a tile no row of this wave sees is masked
    // like any other (its weights are 0), and in the step after the last tile
    // the scores of the stale buffer are computed but never used (live ==
    // false).  Loads past the last tile reload the last tile into a buffer no
    // later step reads.
    // P = (t - t_first) & 1, a compile-time constant: K(t+1) is in K buffer
    // 1 - P; K(t+2) goes to K buffer P, loaded in the S region.  The V loads
    // take one of three schedules (VLATE: in the P V region, so that each
    // load has a whole region to land in and a tile's loads spread over both
    // regions):
    // - two V buffers (head dims up to 128, and bias instances): V(t) is in
    //   V buffer P, V(t+1) is loaded into V buffer 1 - P in the S region, and
    //   the barrier at the end of the step publishes it with K(t+2);
    // - D = 512 (PAIR, VLATE), whose steps already have a barrier between the
    //   regions, the pair exchange: V(t+1) is loaded into V buffer 1 - P in
    //   the P V region, and the next step's exchange barrier publishes it;
    // - three V buffers (V3, VLATE: D 192 and 256 without a bias): V(t) is in
    //   V buffer VB = (t - t_first) % 3 (the steps come in sixes, so that it
    //   is a compile-time constant too), and step t loads V(t+2) in its P V
    //   region into the buffer V(t-1) held; the barrier at the end of step
    //   t+1 publishes it, with no barrier between the regions.
    auto step = [&](int t, f32x16_t (&sc)[KB], f32x16_t (&sn)[KB], auto parity, auto vbuf) {
      constexpr int P = decltype(parity)::value, VB = decltype(vbuf)::value;
      const bool has_next = t < t_last;
      const int tk = ahead(t, 2), tv = ahead(t, V3 ? 2 : 1);
      uint4 pb[KB * 2];
      // the first K operands of the S region, then the rescale for tile t (its
      // factor is known since the last step), so that the interleaved regions
      // are straight-line code
      const uint16_t* const kl = kbuf_at(1 - P);
      uint4 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = kread_at(kl, i, kx(i));
      rescale(alpha_cur);
      uint4 kc[KB + 1];  // 4-bit K: the group-constant operands, A per key block and B
#pragma unroll
      for (int kb = 0; kb <= KB; ++kb) {
        if constexpr (Q4) kc[kb] = kb < KB ? q4_kc_read(kl, kb) : q4_qsum();
        else kc[kb] = make_uint4(0, 0, 0, 0);
      }
      uint2 bw[KB * 4];
      const TileSrc vsrc = tile_src(vg, tv, true);
      uint16_t* const vdst = vbuf_at(V3 ? (VB + 2) % 3 : 1 - P);
      // Q4 with every wave loading: issue this wave's blocks of K(t+3) and
      // V(t+2) now; K(t+2) and V(t+1), issued in the last step, are written to
      // LDS at the end of this one
      if constexpr (Q4) {
        if (!q4_pipe) q4_issue(q4s_k[1 - P], q4s_v[1 - P], min(t + 3, t_last), min(t + 2, t_last));
      }
      const float psum = qk_weights(sn, kl, sc, pb, tile_src(kg, tk, false), kbuf_at(P),
                                    vsrc, vdst, BIAS ? bias_src(tk) : i32x4_t{}, bbuf0 + P * BTILE,
                                    bbuf0 + (1 - P) * BTILE, bw, a, kc);
      exchange(sn, true);  // D = 512: also the V(t) barrier
      l_run = l_run * alpha_cur + psum;
      if (!full_tile(t + 1)) mask(sn, t + 1);
      alpha_cur = pv_max(pb, vbuf_at(V3 ? VB : P), sn, has_next, bw, vsrc, vdst);
      if constexpr (Q4) {
        if (!q4_pipe) q4_put(q4s_k[P], q4s_v[P], kbuf_at(P), vdst);
      }
      // VLATE: K(t+2) (and its bias) have landed, and with V3 V(t+1) too; the
      // V loads of this step may be in flight.  Otherwise everything has.
      if constexpr (VLATE) wait_vmem<PV_LOADS>();
      else __builtin_amdgcn_s_waitcnt(0);
      bias_patch(tk, bbuf0 + P * BTILE);
      __syncthreads();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (wave_active) {
      if constexpr (V3) {
        for (int t = t_first; t <= t_last; t += 6) {
          step(t, sA, sB, I0{}, I0{});
          if (t + 1 > t_last) break;
          step(t + 1, sB, sA, I1{}, I1{});
          if (t + 2 > t_last) break;
          step(t + 2, sA, sB, I0{}, I2{});
          if (t + 3 > t_last) break;
          step(t + 3, sB, sA, I1{}, I0{});
          if (t + 4 > t_last) break;
          step(t + 4, sA, sB, I0{}, I1{});
          if (t + 5 > t_last) break;
          step(t + 5, sB, sA, I1{}, I2{});
        }
      } else {
        for (int t = t_first; t <= t_last; t += 2) {
          step(t, sA, sB, I0{}, I0{});
          if (t + 1 <= t_last) step(t + 1, sB, sA, I1{}, I0{});
        }
      }
    } else if constexpr (Q4) {  // no rows: this wave only loads (4-bit tiles)
      if (q4_pipe) {
        // one step ahead: set a holds K(t+2), V(t+1) when an even step starts
        // (issued in the prologue or the last step), set b when an odd one does
        Q4Data q4b_k[QB], q4b_v[QB];
        // (the scheduling barriers keep each set's loads after the stores of
        // the other, so that the stores never wait for loads just issued)
        for (int t = t_first; t <= t_last; t += 2) {
          q4_put(q4a_k, q4a_v, kbuf0, vbuf0 + TILE);
          __builtin_amdgcn_sched_barrier(0);
          q4_issue(q4b_k, q4b_v, min(t + 3, t_last), min(t + 2, t_last));
          __syncthreads();
          if (t + 1 > t_last) break;
          q4_put(q4b_k, q4b_v, kbuf0 + TILE, vbuf0);
          __builtin_amdgcn_sched_barrier(0);
          q4_issue(q4a_k, q4a_v, min(t + 4, t_last), min(t + 3, t_last));
          __syncthreads();
        }
      } else {  // every wave loads, one step ahead, as the row-holding waves do
        for (int t = t_first; t <= t_last; t += 2) {
          q4_issue(q4s_k[1], q4s_v[1], min(t + 3, t_last), min(t + 2, t_last));
          q4_put(q4s_k[0], q4s_v[0], kbuf0, vbuf0 + TILE);
          __syncthreads();
          if (t + 1 > t_last) break;
          q4_issue(q4s_k[0], q4s_v[0], min(t + 4, t_last), min(t + 3, t_last));
          q4_put(q4s_k[1], q4s_v[1], kbuf0 + TILE, vbuf0);
          __syncthreads();
        }
      }
    } else {  // no rows: this wave only loads its share of every tile and
              // meets the same barriers
      for (int t = t_first; t <= t_last; ++t) {
        if constexpr (PERS) {  // the tiles two places on, also into the next block
          if (t + 2 <= t_last || pf_steps) {
            load_tile(kg, ahead(t, 2), kbuf0 + ((t + 2 - t_first + phase0) & 1) * TILE, false);
            load_tile(vg, ahead(t, 2), vbuf0 + ((t + 2 - t_first + phase0) % NVB) * TILE, true);
          }
        } else if (t + 2 <= t_last) {
          load_k(t + 2);
          load_b(t + 2);
          if constexpr (V3) load_v(t + 2);
        }
        if constexpr (!VLATE)
          if (t < t_last) load_v(t + 1);
        exchange(sA, false);
        if constexpr (PAIR)
          if (t < t_last) load_v(t + 1);
        __builtin_amdgcn_s_waitcnt(0);
        if (t + 2 <= t_last) bias_patch(t + 2, bbuf0 + ((t + 2 - t_first) & 1) * BTILE);
        __syncthreads();
      }
    }
    // no direct load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(0);
  };

  // ---- persistent loop (PERS) ------------------------------------------
  // Row blocks w, w + S, ... of this (batch, KV head) run one after another,
  // each through the same prologue and step loop as a single block.  When a
  // block's step loop ends, the next block's Q rows and K(t0), V(t0),
  // K(t0 + 1) are loaded (every LDS buffer is free by then), and the
  // finished block's output is stored while they are in flight; the next
  // prologue waits for them and loads V(t0 + 1).  Every wave runs every block: a wave whose rows lie past the end
  // of a ragged last block computes on repeated rows and stores nothing.
  if constexpr (PERS) {
    static_assert(V3 && !RING && !BIAS && !Q4 && !PAIR, "the persistent loop takes the three-V-buffer pipeline");
    const int S = p.pers_stride;
    const int nblk = __builtin_amdgcn_readfirstlane((p.mblocks - mbr + S - 1) / S);
    // Q rows of block mbx: rows past a ragged block repeat its last row
    // (they are never stored, and a row's arithmetic never depends on the
    // other rows), so that the loads take no branches
    auto load_q_pers = [&](int mbx) {
      const int r0 = mbx * BM, re = min(p.rows, r0 + BM);
      const int m = min(r0 + rb * kRowsPerWave + lr, re - 1);
      const uint16_t* qrow = p.q + ((size_t)(b * p.Hq + hkv * p.G + m % p.G) * p.qL + m / p.G) * DK + qd0;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) qf[dc] = *(const uint4*)(qrow + dc * 16 + lg * 8);
    };
    auto set_block = [&](int mbx) {  // rows, visible keys and tiles of block mbx
      set_rows(mbx);
      set_keys();
      int kb0, ke0;
      block_keys(mbx, kb0, ke0);
      t_first = __builtin_amdgcn_readfirstlane(kb0 / BN);
      t_last = __builtin_amdgcn_readfirstlane((ke0 - 1) / BN);
    };
    {  // V rows past kL in any block's last tile: zeros before the first load
      int kb0, ke0;
      block_keys(mbr + (nblk - 1) * S, kb0, ke0);
      if (ke0 > kb0 && ((ke0 - 1) / BN + 1) * BN > p.kL) {
        uint4* vz = (uint4*)vbuf0;
        for (int i = tid; i < NVB * TILE / 8; i += NW * 64) vz[i] = make_uint4(0, 0, 0, 0);
        __syncthreads();
      }
    }
    for (int j = 0, pf = 0;;) {
      const bool more = j + 1 < nblk;
      int nf = 0, nl = 0;
      if (more) {
        int kb0, ke0;
        block_keys(mbr + (j + 1) * S, kb0, ke0);
        nf = __builtin_amdgcn_readfirstlane(kb0 / BN);
        nl = __builtin_amdgcn_readfirstlane((ke0 - 1) / BN);
      }
      // this block's last two steps load the next block's first two tiles
      // when both blocks have two or more
      pf_steps = more && t_last > t_first && nl > nf;
      nxt_first = nf;
      run_block(pf);
      // every wave's loads have landed (each waited for its own) before any
      // wave writes LDS below: the last steps load into the buffers
      __syncthreads();
      const float lsum = pair_sum(l_run);
      const bool wave_o = wave_active;
      const int wrow0_o = wrow0, rows_end_o = rows_end;
      if (more) {  // the next block: its rows and tiles, its phase, its Q rows (and K(t0), V(t0), K(t0 + 1))
        const int ntiles = t_last - t_first + 1;
        set_block(mbr + (j + 1) * S);
        phase0 = (phase0 + ntiles) % 6;
        load_q_pers(mbr + (j + 1) * S);
        if (!pf_steps) {
          load_k(t_first);
          load_v(t_first);
          if (t_first < t_last) load_k(t_first + 1);
        }
      }
      pf = pf_steps ? 2 : 1;
      // The finished block's output, normalised and rounded, goes through
      // this wave's 32 rows x 144 bytes of the V buffer that holds neither
      // V(t0) nor V(t0 + 1) of the next block (no load targets it until the
      // next block's first step), 64 columns at a time, so that each lane
      // then stores 16 contiguous bytes and each store instruction writes
      // eight whole 128-byte lines instead of 16 bytes in each of 32 rows.
      // A wave's LDS operations run in order, so its reads see its writes
      // and the next chunk's writes follow this chunk's reads.
      if (wave_o) {
        const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;  // a row with no finite score: zeros
        constexpr int TS = 72;                               // LDS row stride, 16-bit elements (144 bytes)
        uint16_t* const tw = vbuf0 + ((phase0 + 2) % NVB) * TILE + wave * (32 * TS);
        const int sr = lane >> 3, sc = 8 * (lane & 7);      // this lane's row (+ 8 s) and column (+ 64 c)
        size_t orow[4];
        bool okr[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int m = wrow0_o + 8 * s + sr;
          okr[s] = m < rows_end_o;
          orow[s] = ((size_t)(b * p.Hq + hkv * p.G + (okr[s] ? m % p.G : 0)) * p.qL + (okr[s] ? m / p.G : 0)) * DV;
        }
#pragma unroll
        for (int c = 0; c < DB / 2; ++c) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int db = 2 * c + h2;
              uint2 w;
              w.x = Elem<DT>::pack2(o[db][4 * q4 + 0] * inv, o[db][4 * q4 + 1] * inv);
              w.y = Elem<DT>::pack2(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv);
              *(uint2*)(tw + lr * TS + 32 * h2 + 8 * q4 + 4 * lg) = w;
            }
          // the four reads first, all waited for at once (left alone, the
          // compiler moves each into its row's conditional store and waits
          // for the LDS once per store)
          i32x4_t v[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) v[s] = *(const i32x4_t*)(tw + (8 * s + sr) * TS + sc);
          asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (okr[s]) *(i32x4_t*)(p.out + orow[s] + 64 * c + sc) = v[s];
        }
      }
      ++j;
      if (!more) break;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) o[db][jj] = 0.f;
      l_run = 0.f;
      m_ref = -INFINITY;
    }
    return;
  }
  run_block(0);

  // ---- epilogue ---------------------------------------------------------
  const float lsum = pair_sum(l_run);
  if (!valid) return;
  int hq_o = hq, qi_o = qi;
  if constexpr (Q4)
    // the 4-bit instances hold their loaded code words, scales and biases
    // across the step loop; left alone the compiler forms the 64-bit output
    // offset before the loop and spills it, so it is formed here instead
    asm volatile("" : "+v"(hq_o), "+v"(qi_o));
  const size_t orow = (size_t)(b * p.Hq + hq_o) * p.qL + qi_o;
  if (!p.partials) {
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;  // a row with no finite score: zeros
    uint16_t* dst = p.out + orow * DV + od0;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        if (db * 32 + 8 * q4 >= DO) continue;  // columns past the value rows
        const int d = db * 32 + 8 * q4 + 4 * lg;
        uint2 w;
        w.x = Elem<DT>::pack2(o[db][4 * q4 + 0] * inv, o[db][4 * q4 + 1] * inv);
        w.y = Elem<DT>::pack2(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv);
        *(uint2*)(dst + d) = w;
      }
  } else {
    const size_t prow = orow * p.nsplit + split;
    float* dst = p.part_o + prow * DV + od0;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        if (db * 32 + 8 * q4 >= DO) continue;  // columns past the value rows
        const int d = db * 32 + 8 * q4 + 4 * lg;
        *(float4*)(dst + d) =
            make_float4(o[db][4 * q4 + 0], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]);
      }
    if (lg == 0 && h == 0) {
      p.part_ml[prow * 2 + 0] = (m_ref == -INFINITY) ? -INFINITY : m_ref * sl2;
      p.part_ml[prow * 2 + 1] = lsum;
    }
  }
}

// LDS per workgroup: 2 K + 2 V tiles of 64 (32 at D = 512) rows of
// lds_row(DK, DV) elements (+ the pair score exchange at D = 512, 4 waves x
// 4 KiB) (+ 2 bias tiles of the workgroup's rows x the tile's keys)
template <int DT, bool RING, bool BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tile_kernel_d64(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kv_tiles(BIAS, 64) * 64 * 128 + (BIAS ? 2 * 128 * 64 : 0)];
  attn_pipe_body<DT, 64, 64, RING, BIAS>(p, lds);
}
template <int DT, bool RING, bool BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tile_kernel_d80(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kv_tiles(BIAS, 80) * 64 * 128 + (BIAS ? 2 * 128 * 64 : 0)];
  attn_pipe_body<DT, 80, 80, RING, BIAS>(p, lds);
}
template <int DT, bool RING, bool BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tile_kernel_d128(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kv_tiles(BIAS, 128) * 64 * 128 + (BIAS ? 2 * 128 * 64 : 0)];
  attn_pipe_body<DT, 128, 128, RING, BIAS>(p, lds);
}
template <int DT, bool RING, bool BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tile_kernel_d192(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kv_tiles(BIAS, 192) * 64 * 256 + (BIAS ? 2 * 128 * 64 : 0)];
  attn_pipe_body<DT, 192, 192, RING, BIAS>(p, lds);
}
// q and k of head dim 192, v and out of 256 (no ring or bias instances)
template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tile_kernel_dk192_dv256(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kv_tiles(false, 192) * 64 * 256];
  attn_pipe_body<DT, 192, 256, false, false>(p, lds);
}
template <int DT, bool RING, bool BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tile_kernel_d256(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kv_tiles(BIAS, 256) * 64 * 256 + (BIAS ? 2 * 128 * 64 : 0)];
  attn_pipe_body<DT, 256, 256, RING, BIAS>(p, lds);
}
// head dim 256, the persistent loop over several row blocks per workgroup
template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tile_kernel_d256_pers(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kv_tiles(false, 256) * 64 * 256];
  attn_pipe_body<DT, 256, 256, false, false, 0, true>(p, lds);
}
template <int DT, bool RING, bool BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tile_kernel_d512(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * 32 * 512 + 2 * 4 * 64 * 16 + (BIAS ? 2 * 64 * 32 : 0)];
  attn_pipe_body<DT, 512, 512, RING, BIAS>(p, lds);
}

// head dim 256 with 4-bit K and V (2 K + 2 V tiles); Q4M as in attn_pipe_body
template <int DT, int Q4M>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tile_kernel_d256_q4(AttnParams p) {
  // 2 K + 2 V tiles, then the K tiles' group-constant operands (2 x 64 keys x
  // 16) and each lane's query group sums (256 lanes x 8)
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * 64 * 256 + 2 * 64 * 16 + 256 * 8];
  attn_pipe_body<DT, 256, 256, false, false, Q4M>(p, lds);
}

// Merge of the per-split partials of each output row.  One workgroup of nw =
// min(kCombineWaves, nsplit) waves per row: wave w takes the row's chunks
// c_lo + w, c_lo + w + nw, ... in ascending order (so that many chunk loads
// are in flight per row), and the wave partials are then added in wave
// order.  The order depends only on nsplit and the row's own chunk range,
// so a row gets the same bits whatever else is in the call.
constexpr int kCombineWaves = 16;

template <int DT, int D>
__global__ __launch_bounds__(64 * kCombineWaves) void combine_kernel(AttnParams p) {
  // columns per lane, at least 4 (one float4); below D = 256 only lanes
  // [0, D / 4) own columns, the others take part in the reductions only
  constexpr int PER = D / 64 >= 4 ? D / 64 : 4;
  constexpr int NW = kCombineWaves;
  const int nw = blockDim.x >> 6;  // waves in this launch, <= NW
  __shared__ float red[NW];
  __shared__ __attribute__((aligned(16))) float part[NW][D];
  __shared__ float lpart[NW];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool cols = lane * PER < D;
  const size_t row = blockIdx.x;
  const int qi = (int)(row % (size_t)p.qL);
  const int pos = p.q_offset + qi;
  const int key_hi = p.causal ? min(pos, p.kL - 1) : p.kL - 1;
  const int key_lo = p.window > 0 ? max(0, pos - p.window + 1) : 0;
  const int c_lo = key_lo / p.split_len, c_hi = key_hi / p.split_len;
  const float* ml = p.part_ml + row * p.nsplit * 2;
  const float* po = p.part_o + row * (size_t)p.nsplit * D + lane * PER;

  // this wave's first kPre chunks (c_lo + wave + k nw) are loaded now, so that
  // their loads fly with the max pass's instead of after it
  constexpr int kPre = 4;
  float4 pre[kPre][PER / 4];
  float2 pml[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int c = c_lo + wave + k * nw;
    pml[k] = make_float2(-INFINITY, 0.f);
    if (c <= c_hi) {
      pml[k] = *(const float2*)(ml + 2 * c);
      if (cols) {
#pragma unroll
        for (int e = 0; e < PER / 4; ++e) pre[k][e] = *(const float4*)(po + (size_t)c * D + 4 * e);
      }
    }
  }

  // the row's largest reference max (max is exact in any order)
  float m = -INFINITY;
  for (int c = c_lo + tid; c <= c_hi; c += 64 * nw) m = fmaxf(m, ml[2 * c]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float M = red[0];
  for (int w = 1; w < nw; ++w) M = fmaxf(M, red[w]);

  // this wave's chunks, ascending
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    // the same chunks in the same order; the first kPre from the registers
    // loaded above
    auto add = [&](float2 mlc, const float4 (&x)[PER / 4]) {
      const float w = (mlc.x == -INFINITY) ? 0.f : fast_exp2(mlc.x - M);
      L += mlc.y * w;
      if (!cols) return;
#pragma unroll
      for (int e = 0; e < PER / 4; ++e) {
        acc[4 * e + 0] += x[e].x * w;
        acc[4 * e + 1] += x[e].y * w;
        acc[4 * e + 2] += x[e].z * w;
        acc[4 * e + 3] += x[e].w * w;
      }
    };
#pragma unroll
    for (int k = 0; k < kPre; ++k)
      if (c_lo + wave + k * nw <= c_hi) add(pml[k], pre[k]);
    for (int c = c_lo + wave + kPre * nw; c <= c_hi; c += nw) {
      float4 x[PER / 4];
      if (cols) {
#pragma unroll
        for (int e = 0; e < PER / 4; ++e) x[e] = *(const float4*)(po + (size_t)c * D + 4 * e);
      }
      add(*(const float2*)(ml + 2 * c), x);
    }
  }
  if (cols) {
#pragma unroll
    for (int e = 0; e < PER; e += 4)
      *(float4*)(&part[wave][lane * PER + e]) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }
  if (lane == 0) lpart[wave] = L;
  __syncthreads();

  // wave 0: the wave partials in wave order, normalise, round
  if (wave != 0 || !cols) return;
  float Lt = 0.f;
  for (int w = 0; w < nw; ++w) Lt += lpart[w];
  const float inv = (Lt > 0.f) ? 1.0f / Lt : 0.f;
  uint16_t* dst = p.out + row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; e += 4) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int w = 0; w < nw; ++w) {
      const float4 x = *(const float4*)(&part[w][lane * PER + e]);
      t.x += x.x;
      t.y += x.y;
      t.z += x.z;
      t.w += x.w;
    }
    uint2 o2;
    o2.x = Elem<DT>::pack2(t.x * inv, t.y * inv);
    o2.y = Elem<DT>::pack2(t.z * inv, t.w * inv);
    *(uint2*)(dst + e) = o2;
  }
}

// The same merge for calls of at most kCombineFew splits: one wave per row
// (four rows per workgroup), every chunk load in flight at once.  The row's
// chunks are taken in ascending order, and each product is rounded before
// it is added, starting from +0: those are exactly the sums of
// combine_kernel when each of its waves holds at most one of the row's
// chunks, which is always the case when a call with one split more would
// launch it (min(kCombineWaves, nsplit) waves).  So a row's bytes do not
// depend on which of the two kernels merges it.
constexpr int kCombineFew = 4;

template <int DT, int D>
__global__ __launch_bounds__(256) void combine_few_kernel(AttnParams p, size_t rows) {
#pragma clang fp contract(off)  // every product rounded on its own, as described above
  constexpr int PER = D / 64 >= 4 ? D / 64 : 4;
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bool cols = lane * PER < D;
  const int qi = (int)(row % (size_t)p.qL);
  const int pos = p.q_offset + qi;
  const int key_hi = p.causal ? min(pos, p.kL - 1) : p.kL - 1;
  const int key_lo = p.window > 0 ? max(0, pos - p.window + 1) : 0;
  const int c_lo = key_lo / p.split_len, c_hi = key_hi / p.split_len;
  const float* ml = p.part_ml + row * p.nsplit * 2;
  const float* po = p.part_o + row * (size_t)p.nsplit * D + lane * PER;

  float mc[kCombineFew], lc[kCombineFew];
  float4 x[kCombineFew][PER / 4];
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kCombineFew; ++i) {
    const int c = c_lo + i;
    mc[i] = -INFINITY;
    lc[i] = 0.f;
    if (c <= c_hi) {
      mc[i] = ml[2 * c];
      lc[i] = ml[2 * c + 1];
      M = fmaxf(M, mc[i]);
      if (cols) {
#pragma unroll
        for (int e = 0; e < PER / 4; ++e) x[i][e] = *(const float4*)(po + (size_t)c * D + 4 * e);
      }
    }
  }
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kCombineFew; ++i) {
      if (c_lo + i > c_hi) break;
      const float w = (mc[i] == -INFINITY) ? 0.f : fast_exp2(mc[i] - M);
      L = L + lc[i] * w;
      if (!cols) continue;
#pragma unroll
      for (int e = 0; e < PER / 4; ++e) {
        acc[4 * e + 0] = acc[4 * e + 0] + x[i][e].x * w;
        acc[4 * e + 1] = acc[4 * e + 1] + x[i][e].y * w;
        acc[4 * e + 2] = acc[4 * e + 2] + x[i][e].z * w;
        acc[4 * e + 3] = acc[4 * e + 3] + x[i][e].w * w;
      }
    }
  }
  if (!cols) return;
  const float inv = (L > 0.f) ? 1.0f / L : 0.f;
  uint16_t* dst = p.out + row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; e += 4) {
    uint2 o2;
    o2.x = Elem<DT>::pack2(acc[e + 0] * inv, acc[e + 1] * inv);
    o2.y = Elem<DT>::pack2(acc[e + 2] * inv, acc[e + 3] * inv);
    *(uint2*)(dst + e) = o2;
  }
}

template <int DT, int D, bool RING, bool BIAS>
hipError_t launch_attention_t(const AttnParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.B * p.Hkv * p.mblocks), (unsigned)p.nsplit, 1);
  if constexpr (D == 64)
    hipLaunchKernelGGL((attn_tile_kernel_d64<DT, RING, BIAS>), grid, dim3(256), 0, stream, p);
  else if constexpr (D == 80)
    hipLaunchKernelGGL((attn_tile_kernel_d80<DT, RING, BIAS>), grid, dim3(256), 0, stream, p);
  else if constexpr (D == 128)
    hipLaunchKernelGGL((attn_tile_kernel_d128<DT, RING, BIAS>), grid, dim3(256), 0, stream, p);
  else if constexpr (D == 192)
    hipLaunchKernelGGL((attn_tile_kernel_d192<DT, RING, BIAS>), grid, dim3(256), 0, stream, p);
  else if constexpr (D == 256)
    hipLaunchKernelGGL((attn_tile_kernel_d256<DT, RING, BIAS>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_tile_kernel_d512<DT, RING, BIAS>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_combine_t(const AttnParams& p, hipStream_t stream) {
  const size_t total = (size_t)p.B * p.Hq * p.qL;
  if (p.nsplit <= kCombineFew) {  // one wave per output row
    hipLaunchKernelGGL((combine_few_kernel<DT, D>), dim3((unsigned)((total + 3) / 4), 1, 1), dim3(256), 0, stream,
                       p, total);
    return hipGetLastError();
  }
  // one workgroup per output row
  const int nw = p.nsplit < kCombineWaves ? p.nsplit : kCombineWaves;
  hipLaunchKernelGGL((combine_kernel<DT, D>), dim3((unsigned)total, 1, 1), dim3(64 * nw), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

template <int D, bool RING, bool BIAS>
hipError_t launch_attention_d(const AttnParams& p, int dtype, hipStream_t stream) {
  return dtype == 0 ? launch_attention_t<0, D, RING, BIAS>(p, stream) : launch_attention_t<1, D, RING, BIAS>(p, stream);
}

template <int D>
hipError_t launch_attention_dd(const AttnParams& p, int dtype, bool ring, hipStream_t stream) {
  if (p.bias) return launch_attention_d<D, false, true>(p, dtype, stream);  // the host never sets both
  return ring ? launch_attention_d<D, true, false>(p, dtype, stream) : launch_attention_d<D, false, false>(p, dtype, stream);
}

hipError_t launch_attention(const AttnParams& p, int D, int Dv, int dtype, bool ring, hipStream_t stream) {
  if (D != Dv) {  // 192 with 256: the host passes neither a ring nor a bias
    if (ring || p.bias || D != 192 || Dv != 256) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(p.B * p.Hkv * p.mblocks), (unsigned)p.nsplit, 1);
    if (dtype == 0) hipLaunchKernelGGL((attn_tile_kernel_dk192_dv256<0>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((attn_tile_kernel_dk192_dv256<1>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  if (p.pers_stride > 0) {  // the host sets it only for D = 256 without ring, bias or key split
    if (D != 256 || ring || p.bias || p.partials) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(p.B * p.Hkv * p.pers_stride), 1, 1);
    if (dtype == 0) hipLaunchKernelGGL((attn_tile_kernel_d256_pers<0>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((attn_tile_kernel_d256_pers<1>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  if (D == 64) return launch_attention_dd<64>(p, dtype, ring, stream);
  if (D == 80) return launch_attention_dd<80>(p, dtype, ring, stream);
  if (D == 128) return launch_attention_dd<128>(p, dtype, ring, stream);
  if (D == 192) return launch_attention_dd<192>(p, dtype, ring, stream);
  if (D == 256) return launch_attention_dd<256>(p, dtype, ring, stream);
  return launch_attention_dd<512>(p, dtype, ring, stream);
}

hipError_t launch_attention_q4(const AttnParams& p, int dtype, hipStream_t stream) {
  const dim3 grid((unsigned)(p.B * p.Hkv * p.mblocks), (unsigned)p.nsplit, 1);
  // at most 32 packed rows: every workgroup has one row-holding wave
  const bool one = p.rows <= kRowsPerWave;
  if (dtype == 0) {
    if (one) hipLaunchKernelGGL((attn_tile_kernel_d256_q4<0, 1>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((attn_tile_kernel_d256_q4<0, 2>), grid, dim3(256), 0, stream, p);
  } else {
    if (one) hipLaunchKernelGGL((attn_tile_kernel_d256_q4<1, 1>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((attn_tile_kernel_d256_q4<1, 2>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const AttnParams& p, int D, int dtype, hipStream_t stream) {
  if (D == 64) return dtype == 0 ? launch_combine_t<0, 64>(p, stream) : launch_combine_t<1, 64>(p, stream);
  if (D == 80) return dtype == 0 ? launch_combine_t<0, 80>(p, stream) : launch_combine_t<1, 80>(p, stream);
  if (D == 128) return dtype == 0 ? launch_combine_t<0, 128>(p, stream) : launch_combine_t<1, 128>(p, stream);
  if (D == 192) return dtype == 0 ? launch_combine_t<0, 192>(p, stream) : launch_combine_t<1, 192>(p, stream);
  if (D == 256) return dtype == 0 ? launch_combine_t<0, 256>(p, stream) : launch_combine_t<1, 256>(p, stream);
  return dtype == 0 ? launch_combine_t<0, 512>(p, stream) : launch_combine_t<1, 512>(p, stream);
}

}  // namespace sdpa
