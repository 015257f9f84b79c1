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
// K/V tiles go from HBM straight into LDS (global_load_lds, 16 bytes per lane: lane l of
// the wave writes bytes [16 l, 16 l + 16) of a 1 KiB LDS block), so no registers hold them
// and nothing is transposed on the way.  Both tiles are row-major [64 keys][D] in LDS with
// the 16-byte chunks of each row XOR-swizzled so that the MFMA operand reads are spread
// over the LDS banks:
//   K (read 16 bytes per lane, 32 rows at a time): chunk ^ (key % min(chunks per row, 16)).
//   bf16 V (read with ds_read_b64_tr_b16, 8 keys x 64 bytes at a time): chunk ^ 4 (key % 4)
//     for d = 128, chunk ^ 4 ((key / 2) % 2) for d = 64.
//   fp32 V (read 4 bytes per lane; the two lane halves read keys 4 apart): chunk ^ 8 * bit 2
//     of the key.
// Rows past Tk are loaded from row Tk - 1 (real, finite data): their scores are replaced by
// -inf and their weights are 0, so they add nothing.
// ---------------------------------------------------------------------------------------

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void g2l16(const unsigned char *g, unsigned char *lds_block) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                   (__attribute__((address_space(3))) void *)lds_block, 16, 0, 0);
}

// ds_read_b64_tr_b16 at LDS byte address `addr`.  Within each group of 16 lanes, lane r
// supplies 4 consecutive 16-bit elements; lane i receives element i % 4 of the chunks of lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4.  Issued as inline assembly: the compiler's own
// form is treated as possibly reading the LDS buffer that the next tile is being copied into,
// and would wait for that copy.  The caller waits for the result with lds_wait().
template <int OFFSET>
__device__ __forceinline__ s16x4 lds_read_tr16(uint32_t addr) {
  static_assert(OFFSET >= 0 && OFFSET < 65536, "ds offset field is 16 bits");
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFFSET));
  return r;
}
// Waits for every outstanding LDS read of this wave; the operands tie the wait to the values
// it guards, so their uses cannot move above it.
__device__ __forceinline__ void lds_wait(s16x4 &a, s16x4 &b, s16x4 &c, s16x4 &d, s16x4 &e, s16x4 &f,
                                         s16x4 &g, s16x4 &h) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h));
}
__device__ __forceinline__ uint32_t lds_addr(const unsigned char *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)p;
}

template <bool BF16, int D>
struct Layout {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int CH = D * ES / 16;      // 16-byte chunks per row
  static constexpr int RB = 64 / CH;          // rows per 1 KiB block
  static constexpr int NBLK = kBc / RB;       // 1 KiB blocks per tile (per tensor)
  static constexpr int TILE_BYTES = kBc * D * ES;
  __device__ static __forceinline__ int ksw(int key) { return key % (CH < 16 ? CH : 16); }
  __device__ static __forceinline__ int vsw(int key) {
    if constexpr (!BF16) return ((key >> 2) & 1) << 3;
    else if constexpr (D == 128) return 4 * (key & 3);
    else return 4 * ((key >> 1) & 1);
  }
};

template <bool BF16, int D, int NW, int MODE>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(BF16 ? 2 : 1)))
fa_fwd_kernel(Params p) {
  using L = Layout<BF16, D>;
  constexpr int ES = L::ES;
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int BPW = L::NBLK / NW;  // 1 KiB blocks each wave copies per tensor per tile
  static_assert(L::NBLK % NW == 0, "blocks per tile must split evenly over the waves");
  // Two LDS buffers as two objects (each [K | V]), so that the compiler can tell the copy into
  // one from the reads of the other and does not wait for the copy before those reads.
  __shared__ __attribute__((aligned(1024))) unsigned char smem0[2 * L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char smem1[2 * L::TILE_BYTES];

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
  int w_begin = 0, w_end = 0;        // this wave's visible tiles
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
  const float *mrow = MODE == 1 && p.mask
                          ? p.mask + (int64_t)b * p.sm_b + (int64_t)head * p.sm_h + (int64_t)row * p.sm_i
                          : nullptr;

  // This lane's part of the tile copy: row (block * RB + lane / CH), stored chunk lane % CH.
  const int cp_row = lane / L::CH, cp_chunk = lane % L::CH;
  auto issue_tile = [&](int t, unsigned char *kl) {
    unsigned char *vl = kl + L::TILE_BYTES;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wid * BPW + i;
      const int r = blk * L::RB + cp_row;
      int key = t * kBc + r;
      key = key < p.Tk ? key : p.Tk - 1;
      g2l16(kbase + (int64_t)key * p.sk_t * ES + ((cp_chunk ^ L::ksw(r)) * 16), kl + blk * 1024);
      g2l16(vbase + (int64_t)key * p.sv_t * ES + ((cp_chunk ^ L::vsw(r)) * 16), vl + blk * 1024);
    }
  };

  // One tile of work: wait-free reads of `kl` (tile t), copy of tile t + 1 into `kn`.
  auto step = [&](int t, const unsigned char *kl, unsigned char *kn) {
    const unsigned char *vl = kl + L::TILE_BYTES;
    if (t + 1 < t_end) issue_tile(t + 1, kn);  // that buffer was released by the last barrier

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
            const int ch = (2 * ds + half) ^ L::ksw(key);
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kl + key * (D * 2) + ch * 16);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ds], acc, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int c = 0; c < D / 8; ++c) {
            const int ch = (half * (D / 8) + c) ^ L::ksw(key);
            const f32x4 a4 = *reinterpret_cast<const f32x4 *>(kl + key * (D * 4) + ch * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[e], qf[4 * c + e], acc, 0, 0, 0);
          }
        }
        sacc[kb] = acc;
      }

      // ---- scores; keys a row cannot see become -inf by select ----
      // MODE 0 (no mask, scale > 0): the row maximum is taken on the raw dot products (scaling
      //   by a positive constant commutes with max and with fp32 rounding), and each weight is
      //   exp2(fma(s, scale log2 e, -m)).
      // MODE 1 (additive mask, or scale <= 0): x = fma(s, scale log2 e, mask log2 e) first.
      const bool full = (int64_t)t * kBc >= full_lo && (int64_t)t * kBc + kBc <= full_hi;
      if constexpr (MODE == 1) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = t * kBc + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            const float mv = (mrow && row_ok && key < p.Tk) ? mrow[(int64_t)key * p.sm_j] : 0.f;
            sacc[kb][i] = __builtin_fmaf(sacc[kb][i], p.scale_log2, mv * kLog2e);
          }
      }
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int64_t key = (int64_t)t * kBc + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            sacc[kb][i] = (key >= r_lo && key < r_hi) ? sacc[kb][i] : -INFINITY;
          }
      }

      // ---- row maximum (exact, so the reduction order is immaterial) ----
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if constexpr (MODE == 0) mx = mx * p.scale_log2;  // -inf stays -inf (scale > 0)
      const float m_new = fmaxf(m_run, mx);
      const float shift = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - shift);

      // ---- weights and this half's partial denominator (fixed pairwise tree) ----
      float pw[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr (MODE == 0)
            pw[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], p.scale_log2, -shift));
          else
            pw[kb][i] = __builtin_amdgcn_exp2f(sacc[kb][i] - shift);
        }
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
        // which are its S^T registers i = 8(c%2) + j of block c/2.  The matching V^T operand
        // comes from two transposing reads: within each 16-lane group, lane r reads 4 d of
        // key 16c + 8e + 4h + r/4, and lane i receives key ... + j (j = 0..3) at one d.
        bf16x8 pb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[c][j] = (__bf16)pw[c >> 1][8 * (c & 1) + j];
        const int r16 = lane & 15, dh = (lane >> 4) & 1;
        const int key_l = 4 * half + (r16 >> 2);      // key offset of this lane's read
        const int d_l = 16 * dh + 4 * (r16 & 3);      // d offset (elements) of this lane's read
        const uint32_t vbase_l = lds_addr(vl) + key_l * (D * 2) + (d_l & 7) * 2;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = db * 32 + d_l;
          // the swizzle depends on key % 4 (d = 128) or (key / 2) % 2 (d = 64), i.e. on key_l only
          const uint32_t a0 = vbase_l + (((d >> 3) ^ L::vsw(key_l)) * 16);
          s16x4 r[8];  // r[2c + e]: keys 16c + 8e + key_l
          r[0] = lds_read_tr16<0 * D * 2>(a0);
          r[1] = lds_read_tr16<8 * D * 2>(a0);
          r[2] = lds_read_tr16<16 * D * 2>(a0);
          r[3] = lds_read_tr16<24 * D * 2>(a0);
          r[4] = lds_read_tr16<32 * D * 2>(a0);
          r[5] = lds_read_tr16<40 * D * 2>(a0);
          r[6] = lds_read_tr16<48 * D * 2>(a0);
          r[7] = lds_read_tr16<56 * D * 2>(a0);
          lds_wait(r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const s16x8 both = __builtin_shufflevector(r[2 * c], r[2 * c + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pb[c],
                                                               oacc[db], 0, 0, 0);
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
              const int ch = (d >> 2) ^ L::vsw(key);
              const float a = *reinterpret_cast<const float *>(vl + key * (D * 4) + ch * 16 + (d & 3) * 4);
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pw[kb][i], oacc[db], 0, 0, 0);
            }
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of tile t + 1 have landed
    __syncthreads();                // ... everyone's have, and buffer `kl` is free again
  };

  if (t_begin < t_end) {
    issue_tile(t_begin, smem0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int t = t_begin; t < t_end; t += 2) {
    step(t, smem0, smem1);
    if (t + 1 < t_end) step(t + 1, smem1, smem0);
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
KernelFn pick_mode(int mode) {
  return mode ? fa_fwd_kernel<BF16, D, NW, 1> : fa_fwd_kernel<BF16, D, NW, 0>;
}

template <bool BF16, int D>
KernelFn pick_nw(int nw, int mode) {
  switch (nw) {
    case 1: return pick_mode<BF16, D, 1>(mode);
    case 2: return pick_mode<BF16, D, 2>(mode);
    default: return pick_mode<BF16, D, 4>(mode);
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
  // MODE 1 when scores need the explicit form: an additive mask, or a scale that is not
  // positive (the raw-maximum shortcut needs scale > 0).
  const int mode = (mask != nullptr || !(scale > 0.f)) ? 1 : 0;
  KernelFn fn = bf16 ? (d == 64 ? pick_nw<true, 64>(nw, mode) : pick_nw<true, 128>(nw, mode))
                     : (d == 64 ? pick_nw<false, 64>(nw, mode) : pick_nw<false, 128>(nw, mode));
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
