// Fused attention kernels for gfx950 (MI355X).
//
// One workgroup = 4 waves x 32 query rows.  Rows are "packed" grouped-query
// rows: packed row r of KV head hk is query position r / G of query head
// hk * G + r % G, so the G query heads that share a KV head sit in one
// workgroup and every K/V tile is staged into LDS once for all of them.
//
// Per K/V tile (BN keys) each wave computes, with 32x32x16 MFMAs,
//   S^T = K Q^T            (A = K rows from LDS, B = Q from registers)
//   online softmax         (one query row per lane pair, fp32, base 2)
//   O^T += V^T P^T         (A = V^T rows from LDS, B = P from registers)
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

// One 16-byte-per-lane direct global->LDS load from sbase + voff bytes
// (sbase uniform, voff per lane): lane l's 16 bytes land at lds + 16 l.
// Issued through inline assembly so that the compiler does not treat it as a
// pending LDS write and wait for it before every later LDS access; the kernel
// waits for these loads itself, before the barrier that publishes the tile
// they fill.  M0 (the LDS base of the instruction) is restored afterwards;
// writing M0 needs one wait state before the load.
__device__ __forceinline__ void load_lds16(const void* sbase, uint32_t voff, void* lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds);
  // the 64-bit base, moved to scalar registers half by half; readfirstlane
  // returns int, so each half goes through uint32_t (no sign extension)
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const uint64_t sa = ((uint64_t)hi << 32) | (uint64_t)lo;
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sa), "s"(base));
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

// Lazy rescaling: a row's reference max moves only when a tile's max exceeds
// it by more than this many binary orders of magnitude, so exp2 arguments stay
// <= kRescaleLog2 (weights <= 256, well inside the fp16/bf16 range) and the
// output accumulator is rescaled only on those rare tiles.  The result is the
// same softmax; only rounding differs.
constexpr float kRescaleLog2 = 8.f;

template <int DT, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tile_kernel(AttnParams p) {
  constexpr int DS = d_split(D);      // waves per 32-row block
  constexpr int DH = D / DS;          // head-dim slice of one wave (256)
  constexpr int RB = kWaves / DS;     // 32-row blocks per workgroup
  constexpr int BM = block_rows(D);   // rows per workgroup
  constexpr int BN = tile_keys(D);
  constexpr int ROWCH = D / 8;        // 16-byte chunks per K row
  constexpr int KTILE = BN * D;       // K tile: rows of D elements, chunks XOR-swizzled
  constexpr int VTILE = BN * D;       // V tile: key rows of D elements, chunks swizzled
  constexpr int DC = DH / 16;         // MFMA steps over this wave's d in S^T
  constexpr int DB = DH / 32;         // 32-wide d blocks of this wave's O^T
  constexpr int KB = BN / 32;         // 32-key blocks of S^T
  constexpr int KLOADS = BN * D * 2 / 1024 / kWaves;  // 1 KiB direct loads per wave
  constexpr int XCH = DS > 1 ? kWaves * 64 * 16 : 0;  // floats: partial-score exchange
  static_assert(BM == RB * kRowsPerWave, "row blocks");
  static_assert(KLOADS * kWaves * 1024 == BN * D * 2, "K loads must cover the tile");
  static_assert(ROWCH <= 64 && 64 % ROWCH == 0, "a K row must fit one wave load");

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (KTILE + VTILE) + 2 * XCH];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int rb = wave % RB;  // this wave's 32-row block
  const int dh = wave / RB;  // this wave's slice of the head dimension

  // ---- work item: (b, kv head) x row block x key split -------------------
  const int nheads = p.B * p.Hkv;
  const int head = blockIdx.x % nheads;
  const int mbr = blockIdx.x / nheads;
  // causal: later row blocks see more keys; dispatch them first
  const int mb = p.causal ? (p.mblocks - 1 - mbr) : mbr;
  const int split = blockIdx.y;
  const int b = head / p.Hkv, hk = head % p.Hkv;

  const int row0 = mb * BM;
  const int rows_end = min(p.rows, row0 + BM);
  const int wrow0 = row0 + rb * kRowsPerWave;
  const bool wave_active = wrow0 < rows_end;
  const int my = wrow0 + lr;
  const bool valid = my < rows_end;
  const int qi = valid ? my / p.G : 0;
  const int hq = hk * p.G + (valid ? my % p.G : 0);
  const int pos = p.q_offset + qi;
  const int wp_lo = p.q_offset + wrow0 / p.G;
  const int wp_hi = p.q_offset + (min(rows_end, wrow0 + kRowsPerWave) - 1) / p.G;

  // keys any row of this workgroup may see, clipped to the split
  int kbeg = 0, kend = p.kL;
  {
    const int bp_lo = p.q_offset + row0 / p.G;
    const int bp_hi = p.q_offset + (rows_end - 1) / p.G;
    if (p.causal) kend = min(kend, bp_hi + 1);
    if (p.window > 0) kbeg = max(0, bp_lo - p.window + 1);
    if (p.partials) {
      kbeg = max(kbeg, split * p.split_len);
      kend = min(kend, (split + 1) * p.split_len);
    }
  }
  if (kbeg >= kend) return;  // whole workgroup: no row has a key in this split
  const int t_first = kbeg / BN, t_last = (kend - 1) / BN;

  const size_t kv_off = (size_t)(b * p.Hkv + hk) * (size_t)p.kL * D;
  const uint16_t* __restrict__ kg = p.k + kv_off;
  const uint16_t* __restrict__ vg = p.v + kv_off;

  // ---- Q fragments: B operand of S^T = K Q^T,
  //      lane (lr, lg) holds d = dh * DH + 16 dc + 8 lg + 0..7 of its row
  uint4 qf[DC];
  {
    const uint16_t* qrow = p.q + ((size_t)(b * p.Hq + hq) * p.qL + qi) * D + dh * DH;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[dc] = valid ? *(const uint4*)(qrow + dc * 16 + lg * 8) : make_uint4(0, 0, 0, 0);
  }

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float m_ref = -INFINITY;  // reference max of this row's raw scores (moves lazily)
  float l_run = 0.f;        // this lane's share of the row's weight sum

  // ---- per-lane LDS operand offsets (elements), loop invariant -------------
  // K operand (key row kb*32 + lr, 16-byte chunk 2 dc + lg of this wave's d
  // slice): with r = lr & 15 the swizzled chunk is
  //   (lg ^ (r & 1)) + 2 ((dc & 8) | ((dc & 7) ^ (r >> 1)))
  // so eight per-lane offsets plus compile-time immediates cover all (kb, dc)
  int koff[8];
  {
    const int r = lr & 15;
    const int base = lr * D + dh * DH + 8 * (lg ^ (r & 1));
#pragma unroll
    for (int j = 0; j < 8; ++j) koff[j] = base + 16 * (j ^ (r >> 1));
  }
  // V^T operand by transposing reads of the key-major V tile.  Lane l
  // (group g = l / 16, a = l % 4, t = (l % 16) / 4) points at key
  // 16 kh + 8 h + kq, kq = 4 (g / 2) + t, columns dh*DH + 32 db + 16 (g & 1)
  // + 4 a; half h = 0, 1 give the MFMA k slots 0-3 and 4-7, i.e. keys
  // 16 kh + 4 lg + 0..3 and 16 kh + 8 + 4 lg + 0..3, as P holds them.  V
  // rows store 16-byte chunk c at c ^ ((key & 7) << 2); key & 7 == kq, so
  // the swizzle only flips bits 5-7 of the column offset: db ^ kq.
  int vlane;
  {
    const int g = lane >> 4, kq = 4 * (g >> 1) + ((lane >> 2) & 3);
    vlane = kq * D + dh * DH + 32 * kq + 16 * (g & 1) + 4 * (lane & 3);
  }
  auto kaddr = [&](int kb, int dc) {  // element offset inside a K tile
    return koff[dc & 7] + 16 * (dc & 8) + kb * 32 * D;
  };
  auto vaddr = [&](int kh, int db) {  // element offset inside a V tile (half 0)
    return (vlane ^ (32 * db)) + 16 * kh * D;
  };

  // ---- tile staging ------------------------------------------------------
  // K and V: direct global->LDS loads, 1 KiB per wave instruction (lane l
  // writes bytes 16 l .. 16 l + 15 of it), key rows of D elements.  In K,
  // chunk c of row r sits at chunk position c ^ (r & 15), so the 32 rows one
  // K operand read touches fall in distinct banks; in V at c ^ ((r & 7) << 2),
  // which spreads the 8 rows x 64 bytes of one transposing read over all
  // banks.  Rows past kL load row kL - 1: those keys are masked, P is 0.
  auto load_tile = [&](int t, int buf) {
    const int ts = t * BN;
    uint16_t* kl = lds + buf * (KTILE + VTILE);
    uint16_t* vl = kl + KTILE;
    const uint16_t* kt = kg + (size_t)ts * D;  // tile bases: uniform
    const uint16_t* vt = vg + (size_t)ts * D;
    const int nrow = p.kL - ts;                // key rows of this tile inside kL
    auto kvload = [&](int n, bool clamp) {
      const int cb = wave * KLOADS + n;  // 1 KiB block of the tile
      const int row = cb * (64 / ROWCH) + lane / ROWCH;
      const int pch = lane % ROWCH;      // chunk position this lane writes
      const int r = clamp ? min(row, nrow - 1) : row;
      load_lds16(kt, (uint32_t)(r * D + (pch ^ (row & 15)) * 8) * 2u, kl + cb * 512);
      load_lds16(vt, (uint32_t)(r * D + (pch ^ ((row & 7) << 2)) * 8) * 2u, vl + cb * 512);
    };
    if (nrow >= BN) {
#pragma unroll
      for (int n = 0; n < KLOADS; ++n) kvload(n, false);
    } else {  // the last, partial tile
#pragma unroll
      for (int n = 0; n < KLOADS; ++n) kvload(n, true);
    }
  };

  load_tile(t_first, 0);
  __builtin_amdgcn_s_waitcnt(0);  // direct loads have landed in LDS
  __syncthreads();

  const float sl2 = p.sl2;
  for (int t = t_first; t <= t_last; ++t) {
    const int cur = (t - t_first) & 1;
    if (t < t_last) load_tile(t + 1, cur ^ 1);

    const int ts = t * BN, te = ts + BN - 1;
    // wave-uniform; equal for the DS waves that share a row block
    const bool skip = !wave_active || (p.causal && ts > wp_hi) ||
                      (p.window > 0 && te < wp_lo - p.window + 1);
    const uint16_t* kl = lds + cur * (KTILE + VTILE);
    const uint16_t* vl = kl + KTILE;

    // S^T = K Q^T over this wave's d slice: the KB accumulator chains are
    // interleaved (consecutive MFMAs are independent) and K operands are read
    // PF MFMAs ahead; the scheduling barriers keep that order
    f32x16_t s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
    if (!skip) {
      constexpr int NQK = KB * DC, PF = 4;
      auto kread = [&](int n) { return *(const uint4*)(kl + kaddr(n % KB, n / KB)); };
      uint4 a[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) a[i] = kread(i);
#pragma unroll
      for (int n = 0; n < NQK; ++n) {
        const uint4 cur_a = a[n % PF];
        if (n + PF < NQK) a[n % PF] = kread(n + PF);
        s[n % KB] = Elem<DT>::mfma(cur_a, qf[n / KB], s[n % KB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (DS > 1) {
      // the two waves of a row block hold the scores of the two halves of d:
      // swap them through LDS and add (a + b == b + a, so both waves end up
      // with bitwise identical scores and run identical softmax arithmetic)
      float* xch = (float*)(lds + 2 * (KTILE + VTILE));
      if (!skip) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(float4*)(xch + (wave * 4 + q4) * 256 + lane * 4) =
              make_float4(s[0][4 * q4 + 0], s[0][4 * q4 + 1], s[0][4 * q4 + 2], s[0][4 * q4 + 3]);
      }
      __syncthreads();
      if (!skip) {
        const int partner = wave ^ RB;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 x = *(const float4*)(xch + (partner * 4 + q4) * 256 + lane * 4);
          s[0][4 * q4 + 0] += x.x;
          s[0][4 * q4 + 1] += x.y;
          s[0][4 * q4 + 2] += x.z;
          s[0][4 * q4 + 3] += x.w;
        }
      }
    }
    if (!skip) {
      const bool full = (te < p.kL) && (!p.causal || te <= wp_lo) &&
                        (p.window == 0 || ts >= wp_hi - p.window + 1);
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = ts + kb * 32 + 8 * (j >> 2) + 4 * lg + (j & 3);
            const bool vis = key < p.kL && (!p.causal || key <= pos) &&
                             (p.window == 0 || pos - key < p.window);
            s[kb][j] = vis ? s[kb][j] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
      mx = pair_max(mx);
      // move the reference max only when this tile's max is far above it
      const bool upd = mx * sl2 > m_ref * sl2 + kRescaleLog2;
      const float alpha =
          upd ? ((m_ref == -INFINITY) ? 0.f : fast_exp2((m_ref - mx) * sl2)) : 1.f;
      m_ref = upd ? mx : m_ref;
      const float msc = (m_ref == -INFINITY) ? 0.f : m_ref * sl2;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float e = fast_exp2(s[kb][j] * sl2 - msc);
          s[kb][j] = e;
          psum += e;
        }
      l_run = l_run * alpha + psum;
      // x * 1 == x: skip the rescale when no row of the wave moved its reference
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
      }

      // O^T += V^T P^T over this wave's d slice: KB * 2 key halves x DB d
      // blocks, V^T operands read two MFMAs ahead
      uint4 pb[KB * 2];
#pragma unroll
      for (int kh = 0; kh < KB * 2; ++kh) {
        const int kb = kh >> 1, h = kh & 1;
        pb[kh].x = Elem<DT>::pack2(s[kb][8 * h + 0], s[kb][8 * h + 1]);
        pb[kh].y = Elem<DT>::pack2(s[kb][8 * h + 2], s[kb][8 * h + 3]);
        pb[kh].z = Elem<DT>::pack2(s[kb][8 * h + 4], s[kb][8 * h + 5]);
        pb[kh].w = Elem<DT>::pack2(s[kb][8 * h + 6], s[kb][8 * h + 7]);
      }
      constexpr int NPV = KB * 2 * DB, PF = 4;
      auto vread = [&](int n) {
        const uint16_t* a = vl + vaddr(n / DB, n % DB);
        const uint2 lo = read_tr(a), hi = read_tr(a + 8 * D);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      };
      uint4 bv[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) bv[i] = vread(i);
#pragma unroll
      for (int n = 0; n < NPV; ++n) {
        const uint4 cur_b = bv[n % PF];
        if (n + PF < NPV) bv[n % PF] = vread(n + PF);
        o[n % DB] = Elem<DT>::mfma(cur_b, pb[n / DB], o[n % DB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    __builtin_amdgcn_s_waitcnt(0);  // direct loads of the next tile have landed
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------
  const float lsum = pair_sum(l_run);
  if (!valid) return;
  const size_t orow = (size_t)(b * p.Hq + hq) * p.qL + qi;
  if (!p.partials) {
    const float inv = 1.0f / lsum;
    uint16_t* dst = p.out + orow * D + dh * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = db * 32 + 8 * q4 + 4 * lg;
        uint2 w;
        w.x = Elem<DT>::pack2(o[db][4 * q4 + 0] * inv, o[db][4 * q4 + 1] * inv);
        w.y = Elem<DT>::pack2(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv);
        *(uint2*)(dst + d) = w;
      }
  } else {
    const size_t prow = orow * p.nsplit + split;
    float* dst = p.part_o + prow * D + dh * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = db * 32 + 8 * q4 + 4 * lg;
        *(float4*)(dst + d) =
            make_float4(o[db][4 * q4 + 0], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]);
      }
    if (lg == 0 && dh == 0) {
      p.part_ml[prow * 2 + 0] = (m_ref == -INFINITY) ? -INFINITY : m_ref * sl2;
      p.part_ml[prow * 2 + 1] = lsum;
    }
  }
}

// Merge of the per-split partials of each output row, in ascending split
// order over exactly the splits that hold the row's visible keys.  One wave
// per row; every lane recomputes the row's max and sum the same way.
template <int DT, int D>
__global__ __launch_bounds__(256) void combine_kernel(AttnParams p) {
  constexpr int PER = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + wave;
  const size_t total = (size_t)p.B * p.Hq * p.qL;
  if (row >= total) return;
  const int qi = (int)(row % (size_t)p.qL);
  const int pos = p.q_offset + qi;
  const int key_hi = p.causal ? min(pos, p.kL - 1) : p.kL - 1;
  const int key_lo = p.window > 0 ? max(0, pos - p.window + 1) : 0;
  const int c_lo = key_lo / p.split_len, c_hi = key_hi / p.split_len;

  const float* ml = p.part_ml + row * p.nsplit * 2;
  float M = -INFINITY;
  for (int c = c_lo; c <= c_hi; ++c) M = fmaxf(M, ml[2 * c]);
  float L = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  if (M != -INFINITY) {
    for (int c = c_lo; c <= c_hi; ++c) {
      const float mc = ml[2 * c];
      const float w = (mc == -INFINITY) ? 0.f : fast_exp2(mc - M);
      L += ml[2 * c + 1] * w;
      const float* po = p.part_o + (row * p.nsplit + c) * D + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; e += 4) {
        const float4 x = *(const float4*)(po + e);
        acc[e + 0] += x.x * w;
        acc[e + 1] += x.y * w;
        acc[e + 2] += x.z * w;
        acc[e + 3] += x.w * w;
      }
    }
  }
  const float inv = (L > 0.f) ? 1.0f / L : 0.f;
  uint16_t* dst = p.out + row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; e += 4) {
    uint2 w;
    w.x = Elem<DT>::pack2(acc[e + 0] * inv, acc[e + 1] * inv);
    w.y = Elem<DT>::pack2(acc[e + 2] * inv, acc[e + 3] * inv);
    *(uint2*)(dst + e) = w;
  }
}

template <int DT, int D>
hipError_t launch_attention_t(const AttnParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.B * p.Hkv * p.mblocks), (unsigned)p.nsplit, 1);
  hipLaunchKernelGGL((attn_tile_kernel<DT, D>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_combine_t(const AttnParams& p, hipStream_t stream) {
  const size_t total = (size_t)p.B * p.Hq * p.qL;
  const dim3 grid((unsigned)((total + 3) / 4), 1, 1);
  hipLaunchKernelGGL((combine_kernel<DT, D>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int D, int dtype, hipStream_t stream) {
  if (D == 256) return dtype == 0 ? launch_attention_t<0, 256>(p, stream) : launch_attention_t<1, 256>(p, stream);
  return dtype == 0 ? launch_attention_t<0, 512>(p, stream) : launch_attention_t<1, 512>(p, stream);
}

hipError_t launch_combine(const AttnParams& p, int D, int dtype, hipStream_t stream) {
  if (D == 256) return dtype == 0 ? launch_combine_t<0, 256>(p, stream) : launch_combine_t<1, 256>(p, stream);
  return dtype == 0 ? launch_combine_t<0, 512>(p, stream) : launch_combine_t<1, 512>(p, stream);
}

}  // namespace sdpa
