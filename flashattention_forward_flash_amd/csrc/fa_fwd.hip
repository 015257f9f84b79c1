// fa_fwd.hip -- tiled FlashAttention forward for AMD MI355X (gfx950, CDNA4) and its C ABI.
//
// What is computed is stated in include/fa.h ("FlashAttention forward in C", tinyllm L9.3,
// sections 2.1-2.4; the additive mask of "Fused attention and softmax: fast and exact",
// "What is computed").  This file is the device side and the host-side validation.
//
// Design (gfx950-first):
//  * One workgroup = `rows_per_block` query rows x `heads_per_block` query heads of one KV
//    group; one 64-lane wave per 32 rows of one head.  Each K/V tile is staged in LDS once
//    and used by every wave (so a GQA group shares it).
//  * Key tiles are absolute: tile t = keys [64t, 64t + 64).  The workgroup walks the union of
//    its rows' visible tiles; a wave skips tiles none of its rows can see; a row that cannot
//    see a tile its wave processes gets -inf scores there by select, which leaves its state
//    unchanged (alpha = 1 exactly, weights 0).  Each row's arithmetic is therefore fixed by
//    its own position and data ("FlashAttention forward in C", section 2.4).
//  * Scores are computed transposed, S^T = K Q^T, on MFMA 32x32 (bf16: 32x32x16; fp32:
//    32x32x2): a lane owns one query row (lane % 32) and 16 keys per 32-key block, so the
//    row maximum and sum are in-lane reductions plus one exchange between the two lane
//    halves.  The exchange is commutative, so both halves agree exactly.
//  * The output is accumulated transposed, O^T += V^T P^T: the weights stay in the registers
//    that computed them (the S^T accumulator layout is exactly the B-operand layout of the
//    next MFMA once keys are permuted consistently), and the per-row rescale alpha is
//    lane-local.  For bf16, V is stored transposed (d-major) in LDS with the key permutation
//    applied, so each lane reads its 8 keys as one 16-byte LDS read.
//  * Online softmax in base 2: x = s * scale * log2(e); p = exp2(x - m) on the hardware exp2;
//    alpha = exp2(m_old - m_new), taken as exactly 1 when the maximum does not move and as
//    0 when m_old = -inf (the guards of "Fused attention and softmax", exact definition
//    steps 2 and 5); lse = (m + log2 l) ln 2.
//  * Compiled with -ffp-contract=off: every fused multiply-add is written out, so the same
//    source line gives the same bits on every code path (boundary or interior tile).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "fa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBc = 64;       // keys per tile
constexpr int kRowsWave = 32; // query rows per wave (N of the 32x32 MFMA)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Params {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const float *sinks, *mask;
  int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t;
  int64_t sl_b, sl_h, sm_b, sm_h, sm_i, sm_j;
  int64_t q_offset, window;
  int32_t Tq, Tk, Hq, Hkv;
  int32_t group;           // Hq / Hkv
  int32_t heads_per_block; // query heads per workgroup (divides group)
  int32_t rows_per_block;  // query rows per workgroup
  int32_t n_head_groups;   // group / heads_per_block
  int32_t n_row_tiles;     // ceil(Tq / rows_per_block)
  int32_t n_blocks;
  int32_t causal;
  float scale_log2;        // scale * log2(e)
};

// Visible keys of absolute position pos: [vis_lo, vis_hi) ("FlashAttention forward in C",
// section 2.1, the set V_i; a window of w keys ends at pos).
__device__ __forceinline__ int64_t vis_hi(int64_t pos, const Params &p) {
  return p.causal ? (pos + 1 < p.Tk ? pos + 1 : (int64_t)p.Tk) : (int64_t)p.Tk;
}
__device__ __forceinline__ int64_t vis_lo(int64_t pos, const Params &p) {
  return p.window > 0 ? (pos - p.window + 1 > 0 ? pos - p.window + 1 : 0) : 0;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const uint32_t lo = __builtin_bit_cast(unsigned short, (__bf16)a);
  const uint32_t hi = __builtin_bit_cast(unsigned short, (__bf16)b);
  return lo | (hi << 16);
}

// Maps the launch index to a work index so that consecutive work items (which share a KV
// head and hence K/V tiles) land on the same XCD: blocks are dealt to the 8 XCDs round-robin,
// and each XCD gets one contiguous range of work items.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int q = n >> 3, rem = n & 7;
  return xcd < rem ? xcd * (q + 1) + slot : rem * (q + 1) + (xcd - rem) * q + slot;
}

// ---------------------------------------------------------------------------------------
// LDS layouts.
//  bf16 K: [64 keys][D], 16-byte chunks XOR-swizzled by key % (D/8).
//  bf16 V^T: [D][64 keys], keys permuted within each group of 16 so that the 8 keys one
//    lane feeds to one MFMA are contiguous; 16-byte chunks XOR-swizzled by d % 8.
//  fp32 K: [64 keys][D], 16-byte chunks XOR-swizzled by key % 16.
//  fp32 V: [64 keys][D], d XOR-swizzled by 32 * bit 2 of the key (the two lane halves read
//    keys 4 apart and the same d, so they land in different banks).
// ---------------------------------------------------------------------------------------

// Position of key offset k (0..15) inside its group of 16 in the bf16 V^T layout: the MFMA
// B-operand slot (8 * half + j) of the S^T register that holds key k (see PV below).
__device__ __forceinline__ int vt_pos16(int k) { return 8 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3); }

template <bool BF16, int D, int NW>
struct TileIO {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int NT = NW * 64;
  static constexpr int CH = D * ES / 16;              // 16-byte chunks per row
  static constexpr int K_TASKS = kBc * CH;            // one task = one 16-byte chunk of K
  static constexpr int K_PER = (K_TASKS + NT - 1) / NT;
  // V tasks: bf16 = 4 keys x 8 d (transposed on the way to LDS); fp32 = one 16-byte chunk.
  static constexpr int V_TASKS = BF16 ? (kBc / 4) * (D / 8) : K_TASKS;
  static constexpr int V_PER = (V_TASKS + NT - 1) / NT;
  static constexpr int V_REGS = BF16 ? 4 : 1;         // 16-byte registers per V task
  static constexpr int TILE_BYTES = kBc * D * ES;
  // Register-prefetch the next tile (two LDS buffers) when it fits in 64 VGPRs; otherwise
  // copy each tile straight through one LDS buffer.
  static constexpr bool PIPE = (K_PER + V_PER * V_REGS) <= 16;
  static constexpr int LDS_BYTES = (PIPE ? 4 : 2) * TILE_BYTES;

  u32x4 kr[PIPE ? K_PER : 1];
  u32x4 vr[PIPE ? V_PER * V_REGS : 1];

  __device__ static __forceinline__ u32x4 ld_row(const Params &p, const unsigned char *base, int64_t st,
                                                 int key, int ch) {
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < p.Tk) val = *reinterpret_cast<const u32x4 *>(base + ((int64_t)key * st) * ES + ch * 16);
    return val;  // rows past Tk are zero: 0 * weight 0 stays 0
  }
  __device__ static __forceinline__ u32x4 ld_k(const Params &p, const unsigned char *kbase, int key0, int c) {
    if (c >= K_TASKS) return u32x4{0u, 0u, 0u, 0u};
    return ld_row(p, kbase, p.sk_t, key0 + c / CH, c % CH);
  }
  __device__ static __forceinline__ void st_k(unsigned char *kl, int c, u32x4 val) {
    if (c >= K_TASKS) return;
    const int key = c / CH, ch = c % CH;
    const int sw = BF16 ? (key % CH) : (key & 15);
    *reinterpret_cast<u32x4 *>(kl + key * (D * ES) + ((ch ^ sw) * 16)) = val;
  }
  __device__ static __forceinline__ void ld_v(const Params &p, const unsigned char *vbase, int key0, int task,
                                              u32x4 *out) {
    if constexpr (BF16) {
      const int g4 = task / (D / 8), dch = task % (D / 8);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        out[kk] = task < V_TASKS ? ld_row(p, vbase, p.sv_t, key0 + 4 * g4 + kk, dch) : u32x4{0u, 0u, 0u, 0u};
    } else {
      out[0] = task < V_TASKS ? ld_row(p, vbase, p.sv_t, key0 + task / CH, task % CH) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ static __forceinline__ void st_v(unsigned char *vl, int task, const u32x4 *in) {
    if (task >= V_TASKS) return;
    if constexpr (BF16) {
      const int g4 = task / (D / 8), dch = task % (D / 8);
      const int key0 = 4 * g4;                   // 4 consecutive keys, 8 consecutive d
      const int grp = key0 >> 4, pos = vt_pos16(key0 & 15);
      const int lchunk = 2 * grp + (pos >> 3);    // logical 16-byte chunk of the V^T row
      const int hoff = ((pos >> 2) & 1) * 8;      // which 8 bytes of that chunk
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int dd = (s + dch) & 7;             // rotate to spread LDS banks
        const int d = dch * 8 + dd;
        uint32_t e[4];                            // element dd of each key: word dd/2, half dd%2
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t w = in[kk][dd >> 1];
          e[kk] = (dd & 1) ? (w >> 16) : (w & 0xFFFFu);
        }
        const u32x2 pk = {e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
        *reinterpret_cast<u32x2 *>(vl + d * (kBc * 2) + ((lchunk ^ (d & 7)) * 16) + hoff) = pk;
      }
    } else {
      const int key = task / CH, ch = task % CH;
      const int d = (ch * 4) ^ (((key >> 2) & 1) << 5);
      *reinterpret_cast<u32x4 *>(vl + (key * D + d) * 4) = in[0];
    }
  }

  // PIPE: global -> registers for tile t ...
  __device__ __forceinline__ void load(const Params &p, const unsigned char *kbase, const unsigned char *vbase,
                                       int t, int tid) {
    if constexpr (PIPE) {
#pragma unroll
      for (int r = 0; r < K_PER; ++r) kr[r] = ld_k(p, kbase, t * kBc, tid + r * NT);
#pragma unroll
      for (int r = 0; r < V_PER; ++r) ld_v(p, vbase, t * kBc, tid + r * NT, &vr[r * V_REGS]);
    }
  }
  // ... registers -> LDS
  __device__ __forceinline__ void store(unsigned char *kl, unsigned char *vl, int tid) const {
    if constexpr (PIPE) {
#pragma unroll
      for (int r = 0; r < K_PER; ++r) st_k(kl, tid + r * NT, kr[r]);
#pragma unroll
      for (int r = 0; r < V_PER; ++r) st_v(vl, tid + r * NT, &vr[r * V_REGS]);
    }
  }
  // !PIPE: global -> LDS one task at a time
  __device__ static __forceinline__ void copy(const Params &p, const unsigned char *kbase,
                                              const unsigned char *vbase, int t, int tid,
                                              unsigned char *kl, unsigned char *vl) {
#pragma unroll 4
    for (int r = 0; r < K_PER; ++r) st_k(kl, tid + r * NT, ld_k(p, kbase, t * kBc, tid + r * NT));
#pragma unroll 2
    for (int r = 0; r < V_PER; ++r) {
      u32x4 tmp[V_REGS];
      ld_v(p, vbase, t * kBc, tid + r * NT, tmp);
      st_v(vl, tid + r * NT, tmp);
    }
  }
};

template <bool BF16, int D, int NW, bool MASK>
__global__ void __launch_bounds__(NW * 64) fa_fwd_kernel(Params p) {
  using IO = TileIO<BF16, D, NW>;
  constexpr int ES = IO::ES;
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) unsigned char smem[IO::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, lq = lane & 31;

  // ---- work decode: (b, kv head, row tile, head group) ----
  const int w = xcd_remap(blockIdx.x, p.n_blocks);
  const int hg = w % p.n_head_groups;
  int rest = w / p.n_head_groups;
  const int rti = rest % p.n_row_tiles;
  rest /= p.n_row_tiles;
  const int kvh = rest % p.Hkv;
  const int b = rest / p.Hkv;
  const int rt = p.causal ? p.n_row_tiles - 1 - rti : rti;  // heavy (late) row tiles first

  const int G = p.heads_per_block;
  const int head = kvh * p.group + hg * G + (wid % G);
  const int row0_blk = rt * p.rows_per_block;
  const int row0_wave = row0_blk + (wid / G) * kRowsWave;
  const int row = row0_wave + lq;
  const bool row_ok = row < p.Tq;

  // ---- key-tile ranges ----
  int t_begin = 0, t_end = 0;  // workgroup: union of its rows' visible tiles
  {
    const int last = min(row0_blk + p.rows_per_block, p.Tq) - 1;
    const int64_t lo = vis_lo(p.q_offset + row0_blk, p), hi = vis_hi(p.q_offset + last, p);
    if (hi > lo) { t_begin = (int)(lo / kBc); t_end = (int)((hi + kBc - 1) / kBc); }
  }
  int w_begin = 0, w_end = 0;    // this wave's visible tiles
  int64_t full_lo = 1, full_hi = 0;  // tiles inside [full_lo, full_hi) are visible to all its rows
  if (row0_wave < p.Tq) {
    const int last = min(row0_wave + kRowsWave, p.Tq) - 1;
    const int64_t lo0 = vis_lo(p.q_offset + row0_wave, p), hi1 = vis_hi(p.q_offset + last, p);
    if (hi1 > lo0) { w_begin = (int)(lo0 / kBc); w_end = (int)((hi1 + kBc - 1) / kBc); }
    full_lo = vis_lo(p.q_offset + last, p);
    full_hi = vis_hi(p.q_offset + row0_wave, p);
  }
  const int64_t r_lo = row_ok ? vis_lo(p.q_offset + row, p) : 0;
  const int64_t r_hi = row_ok ? vis_hi(p.q_offset + row, p) : 0;

  // ---- Q of this lane's row, held in registers as the MFMA B operand ----
  const unsigned char *qrow = static_cast<const unsigned char *>(p.q) +
                              ((int64_t)b * p.sq_b + (int64_t)head * p.sq_h + (int64_t)row * p.sq_t) * ES;
  bf16x8 qb[BF16 ? D / 16 : 1];
  float qf[BF16 ? 1 : D / 2];
  if constexpr (BF16) {
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      u32x4 val = {0u, 0u, 0u, 0u};
      if (row_ok) val = *reinterpret_cast<const u32x4 *>(qrow + (ds * 16 + 8 * half) * 2);
      qb[ds] = __builtin_bit_cast(bf16x8, val);
    }
  } else {
    // the two lane halves split d: half h owns d in [h * D/2, (h + 1) * D/2)
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      f32x4 val = {0.f, 0.f, 0.f, 0.f};
      if (row_ok) val = *reinterpret_cast<const f32x4 *>(qrow + (half * (D / 2) + 4 * c) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * c + e] = val[e];
    }
  }

  // ---- online-softmax state: m (base-2 units), this half's partial l, O^T accumulators ----
  float m_run = -INFINITY, l_run = 0.f;
  if (p.sinks) {  // a sink is the first "tile": m = z_h, l = e^0 = 1, a = 0
    m_run = p.sinks[head] * kLog2e;
    l_run = half == 0 ? 1.f : 0.f;
  }
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

  const unsigned char *kbase = static_cast<const unsigned char *>(p.k) +
                               ((int64_t)b * p.sk_b + (int64_t)kvh * p.sk_h) * ES;
  const unsigned char *vbase = static_cast<const unsigned char *>(p.v) +
                               ((int64_t)b * p.sv_b + (int64_t)kvh * p.sv_h) * ES;
  const float *mrow = MASK ? p.mask + (int64_t)b * p.sm_b + (int64_t)head * p.sm_h + (int64_t)row * p.sm_i
                           : nullptr;

  IO io;
  if (IO::PIPE && t_begin < t_end) {
    io.load(p, kbase, vbase, t_begin, tid);
    io.store(smem, smem + IO::TILE_BYTES, tid);
    __syncthreads();
  }
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = IO::PIPE ? (t - t_begin) & 1 : 0;
    unsigned char *kl = smem + buf * 2 * IO::TILE_BYTES;
    unsigned char *vl = kl + IO::TILE_BYTES;
    if constexpr (IO::PIPE) {
      if (t + 1 < t_end) io.load(p, kbase, vbase, t + 1, tid);
    } else {
      IO::copy(p, kbase, vbase, t, tid, kl, vl);
      __syncthreads();
    }

    if (t >= w_begin && t < w_end) {
      // ---- S^T = K Q^T for two 32-key blocks; lane holds key 32kb + 8(i/4) + 4 half + i%4 ----
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const int key = kb * 32 + lq;
        if constexpr (BF16) {
#pragma unroll
          for (int ds = 0; ds < D / 16; ++ds) {
            const int ch = (2 * ds + half) ^ (key % IO::CH);
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kl + key * (D * 2) + ch * 16);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ds], acc, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int c = 0; c < D / 8; ++c) {
            const int ch = (half * (D / 8) + c) ^ (key & 15);
            const f32x4 a4 = *reinterpret_cast<const f32x4 *>(kl + key * (D * 4) + ch * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[e], qf[4 * c + e], acc, 0, 0, 0);
          }
        }
        sacc[kb] = acc;
      }

      // ---- scores in base-2 units; invisible keys -> -inf by select ----
      float x[2][16];
      const bool full = (int64_t)t * kBc >= full_lo && (int64_t)t * kBc + kBc <= full_hi;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t * kBc + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          if constexpr (MASK) {
            const float mv = (row_ok && key < p.Tk) ? mrow[(int64_t)key * p.sm_j] : 0.f;
            x[kb][i] = __builtin_fmaf(sacc[kb][i], p.scale_log2, mv * kLog2e);
          } else {
            x[kb][i] = sacc[kb][i] * p.scale_log2;
          }
        }
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int64_t key = (int64_t)t * kBc + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            x[kb][i] = (key >= r_lo && key < r_hi) ? x[kb][i] : -INFINITY;
          }
      }

      // ---- row maximum (exact, so the reduction order is immaterial) ----
      float mx = x[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float shift = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - shift);

      // ---- weights and this half's partial denominator (fixed pairwise tree) ----
      float pw[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) pw[kb][i] = __builtin_amdgcn_exp2f(x[kb][i] - shift);
      float s8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        s8[j] = (pw[j >> 2][4 * (j & 3)] + pw[j >> 2][4 * (j & 3) + 1]) +
                (pw[j >> 2][4 * (j & 3) + 2] + pw[j >> 2][4 * (j & 3) + 3]);
      const float lsum = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
      l_run = __builtin_fmaf(alpha, l_run, lsum);
      m_run = m_new;

      // ---- rescale O^T (skipped when alpha == 1 in every lane: multiplying by 1 is exact) ----
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }

      // ---- O^T += V^T P^T ----
      if constexpr (BF16) {
        // MFMA c covers keys 16c..16c+15; lane half h supplies keys 16c + 8(j/4) + 4h + j%4,
        // which are its S^T registers i = 8(c%2) + j of block c/2.
        bf16x8 pb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[c][j] = (__bf16)pw[c >> 1][8 * (c & 1) + j];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = db * 32 + lq;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int ch = (2 * c + half) ^ (d & 7);
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vl + d * (kBc * 2) + ch * 16);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], oacc[db], 0, 0, 0);
          }
        }
      } else {
        // MFMA (kb, i) contracts 2 keys: lane half h supplies key 32kb + 8(i/4) + 4h + i%4.
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = db * 32 + lq;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
              const float a = *reinterpret_cast<const float *>(vl + (key * D + (d ^ (((key >> 2) & 1) << 5))) * 4);
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pw[kb][i], oacc[db], 0, 0, 0);
            }
        }
      }
    }

    if (IO::PIPE && t + 1 < t_end) {
      unsigned char *kn = smem + (buf ^ 1) * 2 * IO::TILE_BYTES;
      io.store(kn, kn + IO::TILE_BYTES, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: o = a / l, lse = m + ln l; a row that saw nothing gets 0 and -inf ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    unsigned char *orow = static_cast<unsigned char *>(p.o) +
                          ((int64_t)b * p.so_b + (int64_t)head * p.so_h + (int64_t)row * p.so_t) * ES;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * half;  // registers 4g..4g+3 hold d0..d0+3
        float r4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = oacc[db][4 * g + e] * inv;
        if constexpr (BF16) {
          u32x2 pk = {pack_bf16x2(r4[0], r4[1]), pack_bf16x2(r4[2], r4[3])};
          *reinterpret_cast<u32x2 *>(orow + d0 * 2) = pk;
        } else {
          f32x4 v4 = {r4[0], r4[1], r4[2], r4[3]};
          *reinterpret_cast<f32x4 *>(orow + d0 * 4) = v4;
        }
      }
    if (p.lse && half == 0)
      p.lse[(int64_t)b * p.sl_b + (int64_t)head * p.sl_h + row] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------
// Host side: validation (before any launch or write), geometry, dispatch.
// ---------------------------------------------------------------------------------------

typedef void (*KernelFn)(Params);

template <bool BF16, int D, int NW>
KernelFn pick_mask(bool mask) {
  return mask ? fa_fwd_kernel<BF16, D, NW, true> : fa_fwd_kernel<BF16, D, NW, false>;
}

template <bool BF16, int D>
KernelFn pick_nw(int nw, bool mask) {
  switch (nw) {
    case 1: return pick_mask<BF16, D, 1>(mask);
    case 2: return pick_mask<BF16, D, 2>(mask);
    default: return pick_mask<BF16, D, 4>(mask);
  }
}

bool aligned(const void *ptr, int64_t a) { return (reinterpret_cast<uintptr_t>(ptr) % (uintptr_t)a) == 0; }

// Picks (rows_per_block, heads_per_block): prefer 4 waves with as many heads of one KV group
// as divide the group, and fall back to 2 and then 1 wave per workgroup when that leaves the
// 256 CUs with too few workgroups.  Any choice gives the same bits.
void auto_tiling(int64_t B, int64_t Hkv, int64_t group, int64_t Tq, int32_t *rows, int32_t *heads) {
  for (int nw = 4; nw >= 1; nw /= 2) {
    int g = 1;
    for (int c = nw; c >= 2; c /= 2)
      if (group % c == 0) { g = c; break; }
    const int64_t r = 32 * nw / g;
    const int64_t blocks = B * Hkv * (group / g) * ((Tq + r - 1) / r);
    if (blocks >= 512 || nw == 1) {
      *heads = g;
      *rows = (int32_t)r;
      return;
    }
  }
}

fa_status fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                   int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, float scale,
                   int64_t q_offset, int causal, int64_t window, const float *sinks,
                   const float *mask, const fa_strides *strides, fa_dtype dtype, void *stream,
                   const fa_tiling *tiling) {
  // ---- arguments ----
  if (B < 0 || Hq < 0 || Hkv < 0 || Tq < 0 || Tk < 0 || q_offset < 0 || d <= 0) return FA_EINVAL;
  if (!std::isfinite(scale)) return FA_EINVAL;
  if (Hq > 0 && Hkv == 0) return FA_ESHAPE;
  if (Hkv > Hq || (Hkv > 0 && Hq % Hkv != 0)) return FA_ESHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_EUNSUPPORTED;
  if (d != 64 && d != 128) return FA_EUNSUPPORTED;
  const int64_t rows_total = B * Hq * Tq;
  if (rows_total > 0 && (q == nullptr || o == nullptr)) return FA_EINVAL;
  if (rows_total > 0 && Tk > 0 && (k == nullptr || v == nullptr)) return FA_EINVAL;
  // int32 limits of the kernel's row/key indices and of the 1-D grid
  if (Tq > INT32_MAX - 256 || Tk > INT32_MAX - 256 || q_offset > INT64_MAX / 4 ||
      (window > 0 && window > INT64_MAX / 4))
    return FA_EUNSUPPORTED;

  fa_strides s;
  if (strides) {
    s = *strides;
  } else {
    s.q[0] = Hq * Tq * d; s.q[1] = Tq * d; s.q[2] = d;
    s.k[0] = Hkv * Tk * d; s.k[1] = Tk * d; s.k[2] = d;
    s.v[0] = s.k[0]; s.v[1] = s.k[1]; s.v[2] = s.k[2];
    s.o[0] = s.q[0]; s.o[1] = s.q[1]; s.o[2] = s.q[2];
    s.lse[0] = Hq * Tq; s.lse[1] = Tq;
    s.mask[0] = 0; s.mask[1] = 0; s.mask[2] = Tk; s.mask[3] = 1;
  }
  for (int i = 0; i < 3; ++i)
    if (s.q[i] < 0 || s.k[i] < 0 || s.v[i] < 0 || s.o[i] < 0) return FA_EINVAL;
  if (s.lse[0] < 0 || s.lse[1] < 0) return FA_EINVAL;
  for (int i = 0; i < 4; ++i) if (s.mask[i] < 0) return FA_EINVAL;

  int32_t rows_pb = 0, heads_pb = 0;
  const int64_t group = Hkv > 0 ? Hq / Hkv : 1;
  if (tiling && (tiling->rows_per_block != 0 || tiling->heads_per_block != 0)) {
    rows_pb = tiling->rows_per_block;
    heads_pb = tiling->heads_per_block;
    const int64_t waves32 = (int64_t)rows_pb * heads_pb;
    if (rows_pb <= 0 || heads_pb <= 0 || rows_pb % 32 != 0 || group % heads_pb != 0 ||
        (waves32 != 32 && waves32 != 64 && waves32 != 128))
      return FA_EINVAL;
  }
  if (rows_total == 0) return FA_OK;

  // ---- alignment of the vector loads and stores ----
  const int64_t es = dtype == FA_BF16 ? 2 : 4;
  const int64_t oal = dtype == FA_BF16 ? 8 : 16;
  if (!aligned(q, 16) || !aligned(o, oal)) return FA_EUNSUPPORTED;
  for (int i = 0; i < 3; ++i)
    if ((s.q[i] * es) % 16 != 0 || (s.o[i] * es) % oal != 0) return FA_EUNSUPPORTED;
  if (Tk > 0) {
    if (!aligned(k, 16) || !aligned(v, 16)) return FA_EUNSUPPORTED;
    for (int i = 0; i < 3; ++i)
      if ((s.k[i] * es) % 16 != 0 || (s.v[i] * es) % 16 != 0) return FA_EUNSUPPORTED;
  }
  if (!aligned(lse, 4) || !aligned(sinks, 4) || !aligned(mask, 4)) return FA_EUNSUPPORTED;

  if (rows_pb == 0) auto_tiling(B, Hkv, group, Tq, &rows_pb, &heads_pb);
  const int nw = (int)((int64_t)rows_pb * heads_pb / 32);
  const int64_t n_row_tiles = (Tq + rows_pb - 1) / rows_pb;
  const int64_t n_blocks = B * Hkv * (group / heads_pb) * n_row_tiles;
  if (n_blocks > INT32_MAX) return FA_EUNSUPPORTED;

  Params p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.sinks = sinks; p.mask = mask;
  p.sq_b = s.q[0]; p.sq_h = s.q[1]; p.sq_t = s.q[2];
  p.sk_b = s.k[0]; p.sk_h = s.k[1]; p.sk_t = s.k[2];
  p.sv_b = s.v[0]; p.sv_h = s.v[1]; p.sv_t = s.v[2];
  p.so_b = s.o[0]; p.so_h = s.o[1]; p.so_t = s.o[2];
  p.sl_b = s.lse[0]; p.sl_h = s.lse[1];
  p.sm_b = s.mask[0]; p.sm_h = s.mask[1]; p.sm_i = s.mask[2]; p.sm_j = s.mask[3];
  p.q_offset = q_offset;
  p.window = window;
  p.Tq = (int32_t)Tq; p.Tk = (int32_t)Tk; p.Hq = (int32_t)Hq; p.Hkv = (int32_t)Hkv;
  p.group = (int32_t)group;
  p.heads_per_block = heads_pb;
  p.rows_per_block = rows_pb;
  p.n_head_groups = (int32_t)(group / heads_pb);
  p.n_row_tiles = (int32_t)n_row_tiles;
  p.n_blocks = (int32_t)n_blocks;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * kLog2e;

  const bool bf16 = dtype == FA_BF16;
  const bool has_mask = mask != nullptr;
  KernelFn fn = bf16 ? (d == 64 ? pick_nw<true, 64>(nw, has_mask) : pick_nw<true, 128>(nw, has_mask))
                     : (d == 64 ? pick_nw<false, 64>(nw, has_mask) : pick_nw<false, 128>(nw, has_mask));
  (void)hipGetLastError();  // clear a stale error so the check below reports this launch
  hipLaunchKernelGGL(fn, dim3((unsigned)n_blocks), dim3(nw * 64), 0,
                     static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_EDEVICE;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                 int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, float scale,
                 int64_t q_offset, int causal, int64_t window, const float *sinks,
                 const float *mask, const fa_strides *strides, fa_dtype dtype, void *stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks,
                  mask, strides, dtype, stream, nullptr);
}

fa_status fa_fwd_tiled(const void *q, const void *k, const void *v, void *o, float *lse,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                       float scale, int64_t q_offset, int causal, int64_t window,
                       const float *sinks, const float *mask, const fa_strides *strides,
                       fa_dtype dtype, void *stream, const fa_tiling *tiling) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks,
                  mask, strides, dtype, stream, tiling);
}

const char *fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_EINVAL: return "invalid argument";
    case FA_ESHAPE: return "invalid head shape (Hq must be a positive multiple of Hkv)";
    case FA_EUNSUPPORTED: return "unsupported (d must be 64 or 128; dtype fp32 or bf16; aligned tensors)";
    case FA_EDEVICE: return "device launch failed";
  }
  return "unknown status";
}

}  // extern "C"
