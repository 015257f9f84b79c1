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
//    lane-local.  For bf16, V stays row-major in LDS and each lane gathers its V^T operand
//    with transposing LDS reads (ds_read_b64_tr_b16).
//  * Online softmax in base 2: x = s * scale * log2(e); p = exp2(x - m) on the hardware exp2.
//    With an additive mask (MODE 1) s is q.k + fl(mask * fl(1 / scale)), the mask term being
//    the accumulators' starting value, so x = scale (q.k + mask / scale) log2(e).
//    The reference point m moves only when a tile's maximum exceeds it by more than kLazy;
//    alpha = exp2(m_old - m_new) is then exactly 1 when m does not move and 0 when m_old =
//    -inf (the guards of "Fused attention and softmax", exact definition steps 2 and 5);
//    lse = (m + log2 l) ln 2.  fp32 kernels take the row maximum only when it could move m
//    (Wave::weights).  bf16 kernels take it first and then, per 16-key chunk, compute the
//    weights and issue that chunk's PV MFMAs, which run while the next chunk's weights are
//    computed (Wave::softmax_pv); their denominator l sums the weights as rounded for the PV
//    MFMA.
//  * Compiled with -ffp-contract=off: every fused multiply-add is written out, so the same
//    source line gives the same bits on every code path (boundary or interior tile).
//  * The same kernel serves split-KV (a work item per query tile and key split, its row
//    states merged by fa_merge_kernel), paged K/V (each tile's rows found through a block
//    table), packed sequences and per-sequence lengths (seq_params): they change which tiles
//    a work item visits and where a tile is read from, never the arithmetic of a row.
//  * Kernels: MODE 0 (no mask, scale > 0: raw-maximum shortcut), MODE 1 (additive mask,
//    scale > 0: the score accumulators start at mask / scale, then as MODE 0), MODE 2 (softcap
//    / ALiBi score variants, any mask, and any scale <= 0: explicit scores), and for bf16 4-
//    and 8-wave workgroups MODE 3 (softcap, with or without ALiBi) and MODE 4 (ALiBi alone)
//    without a mask: the same arithmetic as MODE 2 with less code, which lets the 4-wave
//    kernels run two waves per SIMD.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "fa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBc = 64;       // keys per tile
constexpr int kRowsWave = 32; // query rows per wave (N of the 32x32 MFMA)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;  // base-2 headroom before the running maximum is moved
constexpr float kLazyW = 256.f;  // 2^kLazy
#ifndef FA_MASK_SLICE_BLOCK
#define FA_MASK_SLICE_BLOCK 4  // work order of a broadcast mask: slices per block (see Work)
#endif
#ifndef FA_QK_LOOKAHEAD
// QK steps the K operand reads run ahead of the MFMAs (at most 6).  One step ahead measured
// ≈ 0.5–1.8 % faster than two on the 8,192-token causal batch and ≈ 2 % on a 2,044-token bf16
// prefill layer (same bits); three and four were slower.
#define FA_QK_LOOKAHEAD 1
#endif
static_assert(FA_QK_LOOKAHEAD >= 1 && FA_QK_LOOKAHEAD <= 6, "2 reads per step, at most 15 LDS reads in flight");

struct Params {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const float *sinks, *mask;
  int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t;
  int64_t sl_b, sl_h, sm_b, sm_h, sm_i, sm_j;
  int64_t q_offset, window;
  int32_t B, Tq, Tk, Hq, Hkv;
  int32_t group;           // Hq / Hkv
  int32_t heads_per_block; // query heads per workgroup (divides group)
  int32_t rows_per_block;  // query rows per workgroup
  int32_t n_head_groups;   // group / heads_per_block
  int32_t n_row_tiles;     // ceil(Tq / rows_per_block)
  int32_t n_blocks;
  int32_t causal;
  int32_t mask_vec;        // mask rows contiguous and 16-byte aligned: read 4 entries at a time
  int32_t tile_major;      // > 0: blocked order for a mask shared by every (b, h), this many slices per block
  int32_t mask_lds;        // MODE 1: each tile's mask block is staged in LDS (MaskStager)
  float scale_log2;        // scale * log2(e)
  float inv_scale;         // 1 / scale (MODE 1: the mask enters the score accumulators as mask / scale)
  // Split-KV ("FlashAttention forward in C", "Going further": split-KV / Flash-Decoding).
  // n_splits = 0: no split, rows end in o and lse.  Otherwise key split s is the absolute key
  // range [64 s split_tiles, 64 (s + 1) split_tiles); a work item covers one split and writes
  // its rows' online-softmax state (m, l, unnormalised acc) to the workspace, row r of split s
  // at ws_ml[2 (s R + r)] and ws_acc[(s R + r) D] with R = B Hq Tq and r = (b Hq + h) Tq + i.
  // The sink term belongs to split 0, the split that starts at key 0.
  float *ws_acc, *ws_ml;
  int32_t n_splits, split_tiles;
  // Paged K/V ("FlashAttention forward in C", "Key Takeaways": paged attention for decode
  // performs the same tile update on blocks).  block_table != null: k and v are pools of
  // num_blocks blocks of block_size keys (a multiple of 64, so a tile lies in one block);
  // key j of sequence b is row j % block_size of block block_table[b * bt_stride +
  // j / block_size], and the (b) strides sk_b, sv_b step from block to block.
  const int32_t *block_table;
  int64_t bt_stride;
  int32_t block_size, num_blocks;
  // Per-sequence lengths.  seqlens_k: sequence b has seqlens_k[b] keys.  Packed sequences
  // (varlen): cu_seqlens_q / cu_seqlens_k are prefix sums over the sequences of the rows of q,
  // o, lse / of k, v, which are then indexed by token through their t strides (the b strides
  // are not used).  Counts are clamped to [0, Tq] and [0, Tk].  With any per-sequence length,
  // the query rows of sequence b are its last rows: q_offset_b = keys_b - rows_b.
  const int32_t *seqlens_k, *cu_seqlens_q, *cu_seqlens_k;
  int32_t Tq_all;          // Tq of the call (the row stride of the split-KV workspace)
  // Score variants (the candle page's flash attention offers softcap and ALiBi): softcap c > 0
  // turns the logit x = scale q.k into c tanh(x / c); ALiBi adds -slope_h |p_i - j|.  Kernels
  // of MODE 2 apply them: cap_in = scale / c, cap_out = c log2(e) (0: no softcap).
  float cap_in, cap_out;
  const float *alibi;      // [Hq] slopes or null
  int64_t q_start, k_start;  // first token of this sequence in packed q, o, lse / k, v
};

__device__ __forceinline__ int32_t clamp_len(int32_t n, int32_t hi) { return n < 0 ? 0 : (n < hi ? n : hi); }

// The lengths, positions and token offsets of sequence b.
__device__ __forceinline__ Params seq_params(const Params &p, int b) {
  Params s = p;
  if (p.cu_seqlens_q) {
    const int32_t q0 = p.cu_seqlens_q[b];
    s.Tq = clamp_len(p.cu_seqlens_q[b + 1] - q0, p.Tq);
    s.q_start = q0;
    s.sq_b = s.so_b = s.sl_b = 0;
  }
  if (p.cu_seqlens_k) {
    const int32_t k0 = p.cu_seqlens_k[b];
    s.Tk = clamp_len(p.cu_seqlens_k[b + 1] - k0, p.Tk);
    s.k_start = k0;
    s.sk_b = s.sv_b = 0;
  } else if (p.seqlens_k) {
    s.Tk = clamp_len(p.seqlens_k[b], p.Tk);
  }
  if (p.seqlens_k || p.cu_seqlens_q || p.cu_seqlens_k) s.q_offset = (int64_t)s.Tk - s.Tq;
  return s;
}

// Visible keys of absolute position pos: [vis_lo, vis_hi) ("FlashAttention forward in C",
// section 2.1, the set V_i; a window of w keys ends at pos).
__device__ __forceinline__ int64_t vis_hi(int64_t pos, const Params &p) {
  return p.causal ? (pos + 1 < p.Tk ? pos + 1 : (int64_t)p.Tk) : (int64_t)p.Tk;
}
__device__ __forceinline__ int64_t vis_lo(int64_t pos, const Params &p) {
  return p.window > 0 ? (pos - p.window + 1 > 0 ? pos - p.window + 1 : 0) : 0;
}

// Split-KV: the key splits [s_lo, s_hi) that meet the visible keys of position pos, and
// whether that is a single split that alone makes the row's result (with a sink, only split 0
// can: it holds the sink).  Such a row is finished by its split's work item like an unsplit
// row (the merge of one split with weight 2^0 = 1 is the same arithmetic); the others are
// merged.
struct SplitSpan {
  int s_lo, s_hi;
  bool single;
  __device__ __forceinline__ SplitSpan(int64_t pos, const Params &p) {
    const int64_t lo = vis_lo(pos, p), hi = vis_hi(pos, p);  // both in [0, Tk]
    const int64_t kps = (int64_t)p.split_tiles * kBc;         // keys per split (the host caps it near Tk)
    s_lo = s_hi = 0;
    if (hi > lo) {
      s_lo = (int)(lo / kps);
      s_hi = (int)((hi - 1) / kps) + 1;
    }
    single = s_hi == s_lo + 1 && (p.sinks == nullptr || s_lo == 0);
  }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const uint32_t lo = __builtin_bit_cast(unsigned short, (__bf16)a);
  const uint32_t hi = __builtin_bit_cast(unsigned short, (__bf16)b);
  return lo | (hi << 16);
}

// tanh(u) for the softcap: the odd Taylor series through u^13 for |u| < kTanhSeries
// (truncation < 4e-7 relative), 1 - 2 / (e^{2|u|} + 1) above (hardware exp2 and reciprocal;
// saturates to 1), with the sign of u.
constexpr float kTanhSeries = 0.55f;
__device__ __forceinline__ float tanh_series(float a) {  // a = |u| < kTanhSeries
  const float a2 = a * a;
  float poly = 21844.f / 6081075.f;
  poly = __builtin_fmaf(poly, a2, -1382.f / 155925.f);
  poly = __builtin_fmaf(poly, a2, 62.f / 2835.f);
  poly = __builtin_fmaf(poly, a2, -17.f / 315.f);
  poly = __builtin_fmaf(poly, a2, 2.f / 15.f);
  poly = __builtin_fmaf(poly, a2, -1.f / 3.f);
  return __builtin_fmaf(poly * a2, a, a);
}
__device__ __forceinline__ float tanh_f(float u) {
  const float a = fabsf(u);
  const float e = __builtin_amdgcn_exp2f(a * (2.f * kLog2e));
  const float big = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
  return copysignf(a < kTanhSeries ? tanh_series(a) : big, u);
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
// K/V tiles go from HBM straight into LDS (buffer loads that write LDS, 16 bytes per lane:
// lane l of the wave writes bytes [16 l, 16 l + 16) of a 1 KiB LDS block), so no registers
// hold them and nothing is transposed on the way.  Both tiles are row-major [64 keys][D] in LDS with
// the 16-byte chunks of each row XOR-swizzled so that the MFMA operand reads are spread
// over the LDS banks:
//   K (read 16 bytes per lane, 32 rows at a time): chunk ^ (key % min(chunks per row, 16)).
//   bf16 V (read with ds_read_b64_tr_b16, 8 keys x 64 bytes at a time): chunk ^ 4 (key % 4)
//     for d = 128, chunk ^ 4 ((key / 2) % 2) for d = 64.
//   fp32 V (read 4 bytes per lane; the two lane halves read keys 4 apart): chunk ^ 8 * bit 2
//     of the key.
// Rows past Tk read as zeros: their scores are replaced by -inf and their weights are 0.
// ---------------------------------------------------------------------------------------

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Buffer loads that write LDS.  The resource and the builtins exist in the device pass only;
// the host pass (which never runs kernel bodies) sees stand-ins.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t BufRsrc;
// Every resource here is uniform over the wave; taking its words with readfirstlane keeps it
// in SGPRs where the compiler cannot prove that (a resource in VGPRs costs a loop per load).
__device__ __forceinline__ BufRsrc make_rsrc(const unsigned char *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes < INT32_MAX ? bytes : INT32_MAX);
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const int nu = __builtin_amdgcn_readfirstlane((int)n);
  return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)(lo | (hi << 32)), (short)0, nu, 0x00020000 /* raw dwords */);
}
__device__ __forceinline__ void buf_load_lds16(BufRsrc rs, unsigned char *lds_block, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds_block, 16, off, 0, 0, 0);
}
// The same copy as a global load that writes LDS (global_load_lds_dwordx4): cheaper to issue,
// but without a range check, so only for bytes known to lie inside the tensor.
__device__ __forceinline__ void glb_load_lds16(const unsigned char *base, unsigned char *lds_block, uint32_t off) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + off),
                                   (__attribute__((address_space(3))) void *)lds_block, 16, 0, 0);
}
// 16 bytes per lane into registers through a resource (bytes past its range read as zeros)
__device__ __forceinline__ u32x4 buf_load16(BufRsrc rs, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
}
#else
typedef int BufRsrc;
__device__ inline BufRsrc make_rsrc(const unsigned char *, int64_t) { return 0; }
__device__ inline void buf_load_lds16(BufRsrc, unsigned char *, uint32_t) {}
__device__ inline void glb_load_lds16(const unsigned char *, unsigned char *, uint32_t) {}
__device__ inline u32x4 buf_load16(BufRsrc, uint32_t) { return u32x4{0u, 0u, 0u, 0u}; }
#endif


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
// ds_read_b128 at LDS byte address `addr` + OFFSET, issued as inline assembly like the
// transposing read (the wait is placed by the caller).
template <int OFFSET>
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  static_assert(OFFSET >= 0 && OFFSET < 65536, "ds offset field is 16 bits");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFFSET));
  return r;
}
// Waits until at most N of this wave's LDS reads are outstanding.  LDS reads complete in
// order and these code paths issue no scalar-memory reads, so all but the N newest reads have
// landed.  The operands tie the wait to the values it guards, so their uses cannot move
// above it.
template <int N, typename T>
__device__ __forceinline__ void lds_wait(T &a, T &b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}
template <int N, typename T>
__device__ __forceinline__ void lds_wait(T &a, T &b, T &c, T &d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N));
}
template <int N, typename T>
__device__ __forceinline__ void lds_wait(T &a, T &b, T &c, T &d, T &e, T &f, T &g, T &h) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h)
               : "i"(N));
}
// A uniform load of data that no kernel writes while this one runs (the block table), through
// the scalar cache: it is counted by lgkmcnt, not by vmcnt, so it does not wait for the tile
// copies in flight.
__device__ __forceinline__ int32_t load_const(const int32_t *ptr) {
  return *(const __attribute__((address_space(4))) int32_t *)ptr;
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

// ---------------------------------------------------------------------------------------
// Work decode and the key-tile ranges of one workgroup.
// ---------------------------------------------------------------------------------------
struct Work {
  int b, kvh, head_base, row0_blk, split, t_begin, t_end;
  __device__ __forceinline__ Work(const Params &p) : Work(p, (int)blockIdx.x) {}
  // vb: the launch index the work item would have in a one-item-per-workgroup launch
  __device__ __forceinline__ Work(const Params &p, int vb) {
    const int w = xcd_remap(vb, p.n_blocks);
    const int hg = w % p.n_head_groups;
    int rest = w / p.n_head_groups;
    int rti;
    split = 0;
    if (p.tile_major) {
      // A mask shared by every (b, h): work comes in blocks of tile_major slices (a slice = one
      // (split, b, kv head, head group)) by every row tile, slice fastest, so that the
      // workgroups an XCD runs together share both mask rows (same row tile) and K/V tiles
      // (same slice).  `hg` above is the slice's head group.
      const int sb = p.tile_major;
      const int s_in = w / p.n_head_groups % sb;
      rest = w / p.n_head_groups / sb;
      rti = rest % p.n_row_tiles;
      rest = (rest / p.n_row_tiles) * sb + s_in;  // the slice, without its head group
      kvh = rest % p.Hkv;
      rest /= p.Hkv;
      b = rest % p.B;
      rest /= p.B;
      if (p.n_splits > 0) split = rest;
    } else {             // (b, kv head, split, row tile, head group): neighbours share K and V
      rti = rest % p.n_row_tiles;
      rest /= p.n_row_tiles;
      if (p.n_splits > 0) { split = rest % p.n_splits; rest /= p.n_splits; }
      kvh = rest % p.Hkv;
      b = rest / p.Hkv;
    }
    const int rt = p.causal ? p.n_row_tiles - 1 - rti : rti;  // heavy (late) row tiles first
    head_base = kvh * p.group + hg * p.heads_per_block;
    row0_blk = rt * p.rows_per_block;
  }
  // The union of the visible tiles of the workgroup's rows (lo and hi grow with the position),
  // with p the parameters of sequence b.
  __device__ __forceinline__ void set_range(const Params &p) {
    t_begin = t_end = 0;
    if (row0_blk >= p.Tq) return;  // a packed sequence shorter than the call's Tq
    const int last = min(row0_blk + p.rows_per_block, p.Tq) - 1;
    const int64_t lo = vis_lo(p.q_offset + row0_blk, p), hi = vis_hi(p.q_offset + last, p);
    if (hi > lo) { t_begin = (int)(lo / kBc); t_end = (int)((hi + kBc - 1) / kBc); }
    if (p.n_splits > 0) {  // ... within this work item's key split
      t_begin = max(t_begin, split * p.split_tiles);
      t_end = max(t_begin, min(t_end, (split + 1) * p.split_tiles));
    }
  }
};

// ---------------------------------------------------------------------------------------
// One wave: 32 query rows of one head.  Holds the rows' Q (MFMA B operand), the O^T
// accumulators and the online-softmax state, and does the per-tile math.
// ---------------------------------------------------------------------------------------
// DP > 1 (fp32 only): DP waves share one head's 32 rows, each computing the scores and weights
// of every key and the output for its own D / DP of the d range (blocks of 32); every output
// element has the arithmetic of DP = 1, so the bits do not change.
template <bool BF16, int D, int MODE, int DP = 1>
struct Wave {
  using L = Layout<BF16, D>;
  static constexpr int ES = L::ES;
  static constexpr int NDB = D / 32;  // 32-row blocks of O^T
  static constexpr int NOB = NDB / DP;  // ... that this wave computes: dpart * NOB + [0, NOB)
  static_assert(DP == 1 || (!BF16 && NDB % DP == 0), "d parts: fp32 kernels, whole blocks");

  int half, lq, lane, row;
  bool row_ok;
  int r_lo, r_hi;            // this row's visible keys [r_lo, r_hi)
  int w_begin, w_end;        // tiles holding any key visible to the wave's rows
  int64_t full_lo, full_hi;  // tiles inside [full_lo, full_hi) are visible to all its rows
  const float *mrow;
  uint32_t mask_lds_row;     // MODE 1 with a staged mask: this row's place in the LDS block
  float al_slope;            // MODE 2-4: -slope_h log2(e) (0 without ALiBi)
  int64_t pos;               // MODE 2-4: the row's absolute position
  bf16x8 qb[BF16 ? D / 16 : 1];
  float qf[BF16 ? 1 : D / 2];
  float m_run, l_run;        // reference maximum (base-2 units) and this half's partial l
  int dpart;                 // DP > 1: this wave's part of the d range
  f32x16 oacc[NOB];
  f32x16 sacc[2];            // S^T of the current tile; lane holds key 32kb + 8(i/4) + 4 half + i%4
  bf16x8 pb[BF16 ? 4 : 1];   // bf16 weights, the B operand of the PV MFMAs
  float pw[BF16 ? 1 : 2][16];  // fp32 weights (fp32 path)

  __device__ __forceinline__ void init(const Params &p, int b, int head, int row0_wave, int lane_,
                                       bool with_sink, int dpart_ = 0, bool load_q = true) {
    lane = lane_;
    dpart = dpart_;
    half = lane >> 5;
    lq = lane & 31;
    row = row0_wave + lq;
    row_ok = row < p.Tq;
    w_begin = w_end = 0;
    full_lo = 1;
    full_hi = 0;
    if (row0_wave < p.Tq) {
      const int last = min(row0_wave + kRowsWave, p.Tq) - 1;
      const int64_t lo0 = vis_lo(p.q_offset + row0_wave, p), hi1 = vis_hi(p.q_offset + last, p);
      if (hi1 > lo0) { w_begin = (int)(lo0 / kBc); w_end = (int)((hi1 + kBc - 1) / kBc); }
      full_lo = vis_lo(p.q_offset + last, p);
      full_hi = vis_hi(p.q_offset + row0_wave, p);
    }
    // clamped to [0, Tk] so they fit 32 bits
    r_hi = row_ok ? (int)vis_hi(p.q_offset + row, p) : 0;
    r_lo = row_ok ? (int)min(vis_lo(p.q_offset + row, p), (int64_t)r_hi) : 0;
    if constexpr (MODE >= 2) {
      al_slope = p.alibi ? -p.alibi[head] * kLog2e : 0.f;
      pos = p.q_offset + row;
    }
    mrow = (MODE == 1 || MODE == 2) && p.mask
               ? p.mask + (int64_t)b * p.sm_b + (int64_t)head * p.sm_h + (int64_t)row * p.sm_i
               : nullptr;

    if (load_q) load_q_rows(p, b, head, row0_wave);
    m_run = row_ok ? -INFINITY : 0.f;  // rows past Tq are never written
    l_run = 0.f;
    if (p.sinks && with_sink) {  // a sink is the first "tile": m = z_h, l = e^0 = 1, a = 0
      m_run = p.sinks[head] * kLog2e;
      l_run = half == 0 ? 1.f : 0.f;
    }
#pragma unroll
    for (int db = 0; db < NOB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  }

  // Q rows row0_wave + lq of head `head` into the MFMA operand registers (zeros past Tq); the
  // rest of the wave's state is left alone (a persistent workgroup loads the next work item's
  // Q during the current item's last tile).
  __device__ __forceinline__ void load_q_rows(const Params &p, int b, int head, int row0_wave) {
    const int qr = row0_wave + (lane & 31);
    const bool ok = qr < p.Tq;
    const unsigned char *qrow = static_cast<const unsigned char *>(p.q) +
                                ((int64_t)b * p.sq_b + (int64_t)head * p.sq_h + (p.q_start + qr) * p.sq_t) * ES;
    const int hf = lane >> 5;
    if constexpr (BF16) {
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (ok) val = *reinterpret_cast<const u32x4 *>(qrow + (ds * 16 + 8 * hf) * 2);
        qb[ds] = __builtin_bit_cast(bf16x8, val);
      }
    } else {
      // the two lane halves split d: half h owns d in [h * D/2, (h + 1) * D/2)
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        f32x4 val = {0.f, 0.f, 0.f, 0.f};
        if (ok) val = *reinterpret_cast<const f32x4 *>(qrow + (hf * (D / 2) + 4 * c) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[4 * c + e] = val[e];
      }
    }
  }

  __device__ __forceinline__ bool active(int t) const { return t >= w_begin && t < w_end; }

  // S^T = K Q^T for the two 32-key blocks of the tile in `kl`, into `dst`.  The two blocks'
  // MFMA chains are interleaved so that consecutive MFMAs are independent.  PIPE: the K
  // operand reads are issued one step ahead by hand (bf16); otherwise they are left to the
  // compiler, which can then interleave them with other work of the same block.
  template <bool PIPE>
  __device__ __forceinline__ void qk(const unsigned char *kl, f32x16 (&dst)[2]) const {
    qk<PIPE>(kl, dst, [](int) {});
  }
  // `hook(ds)` runs after the operand reads of step ds + 1 are issued (bf16 with PIPE; before
  // the MFMAs otherwise): the caller places the next tile's copies there, spread over the
  // steps, so that the wave never stalls on a full memory-issue queue.
  template <bool PIPE, typename Hook>
  __device__ __forceinline__ void qk(const unsigned char *kl, f32x16 (&dst)[2], Hook &&hook) const {
    if constexpr (MODE != 1) {  // MODE 1: mask_acc() filled them
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[kb][r] = 0.f;
    }
    if constexpr (BF16 && PIPE) {
      // K operand of step ds for both key blocks: row kb * 32 + lq, chunk (2 ds + half) swizzled
      // by the row (key % chunks-per-row is lq % chunks-per-row for both blocks).
      constexpr int NDS = D / 16;
      const uint32_t krow = lds_addr(kl) + lq * (D * 2);
      const int m = L::ksw(lq);
      // ring of KLA + 1 steps of K operands: the reads run KLA steps ahead of the MFMAs
      constexpr int KLA = FA_QK_LOOKAHEAD;
      u32x4 ka[KLA + 1][2];
      auto issue = [&](int ds) {
        const uint32_t a = krow + ((((2 * ds + half) ^ m)) << 4);
        ka[ds % (KLA + 1)][0] = lds_read_b128<0>(a);
        ka[ds % (KLA + 1)][1] = lds_read_b128<32 * D * 2>(a);
      };
#pragma unroll
      for (int ds = 0; ds < KLA; ++ds) issue(ds);
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        u32x4 *kc = ka[ds % (KLA + 1)];
        if (ds + KLA < NDS) issue(ds + KLA);
        hook(ds);
        // reads issued after step ds's: 2 per later step already in flight
        const int ahead = (NDS - 1 - ds) < KLA ? (NDS - 1 - ds) : KLA;
        switch (ahead) {
          case 0: lds_wait<0>(kc[0], kc[1]); break;
          case 1: lds_wait<2>(kc[0], kc[1]); break;
          case 2: lds_wait<4>(kc[0], kc[1]); break;
          case 3: lds_wait<6>(kc[0], kc[1]); break;
          case 4: lds_wait<8>(kc[0], kc[1]); break;
          case 5: lds_wait<10>(kc[0], kc[1]); break;
          default: lds_wait<12>(kc[0], kc[1]); break;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          dst[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kc[kb]), qb[ds], dst[kb], 0, 0, 0);
      }
    } else if constexpr (BF16) {
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) hook(ds);
      const unsigned char *krow = kl + lq * (D * 2);
      const int m = L::ksw(lq);
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + kb * 32 * (D * 2) + (((2 * ds + half) ^ m) * 16));
          dst[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ds], dst[kb], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) hook(ds);
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        f32x4 a4[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int key = kb * 32 + lq;
          const int ch = (half * (D / 8) + c) ^ L::ksw(key);
          a4[kb] = *reinterpret_cast<const f32x4 *>(kl + key * (D * 4) + ch * 16);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            dst[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[kb][e], qf[4 * c + e], dst[kb], 0, 0, 0);
      }
    }
  }

  // fp32: S^T of key block kb alone, by the MFMA chain qk() runs for that block (same
  // operands, same order, so the same bits).
  // `hook(c)` runs before chunk c's MFMAs (the caller spreads its copies there).
  template <typename Hook>
  __device__ __forceinline__ void qk_block(const unsigned char *kl, int kb, f32x16 &dst, Hook &&hook) const {
    static_assert(!BF16, "fp32 score waves");
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[r] = 0.f;
    const int key = kb * 32 + lq;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      hook(c);
      const int ch = (half * (D / 8) + c) ^ L::ksw(key);
      const f32x4 a4 = *reinterpret_cast<const f32x4 *>(kl + key * (D * 4) + ch * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[e], qf[4 * c + e], dst, 0, 0, 0);
    }
  }

  __device__ __forceinline__ bool full(int t) const {
    return (int64_t)t * kBc >= full_lo && (int64_t)t * kBc + kBc <= full_hi;
  }

  // Scores of tile t in base-2 units where needed.
  // MODE 0 (no mask, scale > 0): the scores stay raw dot products; the row maximum is taken on
  //   them (scaling by a positive constant commutes with max and with fp32 rounding) and each
  //   weight is exp2(fma(s, scale log2 e, -m)).
  // MODE 1 (additive mask, scale > 0): the score accumulators start at mask / scale (mask_acc)
  //   and the MFMAs add q.k to them, so y = scale (q.k + mask / scale); from there on, MODE 0.
  // MODE 2-4 (softcap or ALiBi, or scale <= 0): x = [c log2 e tanh(s scale / c) | s scale log2 e]
  //   + dist (-slope log2 e) + mask log2 e (MODE 2 only: 3 and 4 have no mask).
  __device__ __forceinline__ void scores(const Params &p, int t, f32x16 (&sc)[2]) const {
    if constexpr (MODE >= 2) {
      variants(p, t, sc);
      if (MODE != 2 || !p.mask) return;
      float mv[2][16];
      if (mrow && p.mask_vec && t * kBc + kBc <= p.Tk) {
        // registers 4g..4g+3 of a block hold 4 consecutive keys: one 16-byte read
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 m4 = {0.f, 0.f, 0.f, 0.f};
            if (row_ok) m4 = *reinterpret_cast<const f32x4 *>(mrow + t * kBc + kb * 32 + 8 * g + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) mv[kb][4 * g + e] = m4[e];
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = t * kBc + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            mv[kb][i] = (mrow && row_ok && key < p.Tk) ? mrow[(int64_t)key * p.sm_j] : 0.f;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kb][i] = sc[kb][i] + mv[kb][i] * kLog2e;
    }
  }
  // MODE 1: the score accumulators of tile t before its QK MFMAs, mask / scale per entry
  // (entries past the mask's end and rows past Tq: 0).  From the staged LDS block, whose
  // entries the stager already divided (the same product, fl(mask * fl(1 / scale))), or from
  // the mask rows in global memory.
  __device__ __forceinline__ void mask_acc(const Params &p, int t, const unsigned char *ml,
                                           f32x16 (&sc)[2]) const {
    static_assert(MODE == 1, "additive mask in the accumulators");
    if (p.mask_lds) {
      // the row's 64 entries of the staged block: logical 16-byte chunk c of LDS row r sits at
      // chunk c ^ (r % 16); registers 4g..4g+3 of key block kb are chunk 8 kb + 2 g + half
      const uint32_t r = mask_lds_row;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t c = (uint32_t)(kb * 8 + 2 * g + half) ^ (r & 15u);
          const f32x4 m4 = *reinterpret_cast<const f32x4 *>(ml + r * 256u + c * 16u);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[kb][4 * g + e] = m4[e];
        }
      return;
    }
    if (mrow && p.mask_vec && t * kBc + kBc <= p.Tk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 m4 = {0.f, 0.f, 0.f, 0.f};
          if (row_ok) m4 = *reinterpret_cast<const f32x4 *>(mrow + t * kBc + kb * 32 + 8 * g + 4 * half);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[kb][4 * g + e] = m4[e] * p.inv_scale;
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t * kBc + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          sc[kb][i] = ((mrow && row_ok && key < p.Tk) ? mrow[(int64_t)key * p.sm_j] : 0.f) * p.inv_scale;
        }
    }
  }
  // MODE 2-4 before any mask: the capped logit and the ALiBi bias.  The distance |p - key| is
  // |(p - 64 t) - offset| in fp32, exact for distances below 2^24 (the offset of register i is
  // the key's place in the tile).
  __device__ __forceinline__ void variants(const Params &p, int t, f32x16 (&sc)[2]) const {
    const float d0 = (float)(pos - (int64_t)t * kBc);
    auto biased = [&](float x, int kb, int i) {
      const float off = (float)(kb * 32 + 8 * (i >> 2) + (i & 3)) + (half ? 4.f : 0.f);
      return __builtin_fmaf(fabsf(d0 - off), al_slope, x);
    };
    if (MODE == 3 || (MODE == 2 && p.cap_out > 0.f)) {
      // When no argument of the wave reaches the series' bound this tile, tanh_f would take the
      // series everywhere: the exponential branch is left out (same bits).  The largest |s|
      // decides, since |s cap_in| rounds monotonically in |s|.
      float smax = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) smax = fmaxf(smax, fabsf(sc[kb][i]));
      if (__ballot(smax * fabsf(p.cap_in) >= kTanhSeries)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[kb][i] = biased(tanh_f(sc[kb][i] * p.cap_in) * p.cap_out, kb, i);
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float u = sc[kb][i] * p.cap_in;
            sc[kb][i] = biased(copysignf(tanh_series(fabsf(u)), u) * p.cap_out, kb, i);
          }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kb][i] = biased(sc[kb][i] * p.scale_log2, kb, i);
    }
  }
  // Keys this row cannot see become -inf by select (a no-op on tiles that are `full`).
  __device__ __forceinline__ void select(int t, f32x16 (&sc)[2]) const {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t * kBc + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        sc[kb][i] = (key >= r_lo && key < r_hi) ? sc[kb][i] : -INFINITY;
      }
  }

  // fp32 kernels: the tile's weights exp2(x - shift) in base-2 units (the B operand of the PV
  // MFMAs) and this half's partial denominator.
  __device__ __forceinline__ float expw_one(const Params &p, float x, float shift) const {
    if constexpr (MODE <= 1) return __builtin_amdgcn_exp2f(__builtin_fmaf(x, p.scale_log2, -shift));
    else return __builtin_amdgcn_exp2f(x - shift);
  }
  // the partial denominator: the 32 weights summed as a fixed tree
  __device__ __forceinline__ static float wsum(const float (&w)[2][16]) {
    float s8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      s8[j] = (w[j >> 2][4 * (j & 3)] + w[j >> 2][4 * (j & 3) + 1]) +
              (w[j >> 2][4 * (j & 3) + 2] + w[j >> 2][4 * (j & 3) + 3]);
    return ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
  }
  __device__ __forceinline__ float expw(const Params &p, const f32x16 (&sc)[2], float shift) {
    return expw(p, sc, shift, pw);
  }
  __device__ __forceinline__ float expw(const Params &p, const f32x16 (&sc)[2], float shift, float (&wout)[2][16]) {
    static_assert(!BF16, "bf16 kernels take softmax_pv");
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) wout[kb][i] = expw_one(p, sc[kb][i], shift);
    return wsum(wout);
  }

  // The reference point m of the online softmax.  It moves only when the tile's row maximum
  // exceeds it by more than kLazy (base-2 units), or m is still -inf: weights are then
  // exp2(x - m) <= 2^kLazy, and most tiles need no rescale.  The rule depends on the row's own
  // scores only, so a row's bits stay independent of chunking and query tiling.  Returns the
  // new m; `shift` is the point weights are taken against, `alpha` the factor for O^T and l.
  __device__ __forceinline__ float ref_point(const Params &p, const f32x16 (&sc)[2], float &shift,
                                             float &alpha) const {
    // row maximum (exact, so the reduction order is immaterial)
    float mx = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
    // to base-2 units (a positive factor commutes with max and with fp32 rounding; -inf stays)
    if constexpr (MODE <= 1) mx = mx * p.scale_log2;
    // The row maximum exceeds m + kLazy exactly when one lane half's maximum does, so the
    // exchange between the halves is only needed when some lane's does.
    float m_new = m_run;
    if (__ballot(mx > m_run + kLazy)) {
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m_new = (mx > m_run + kLazy) ? mx : m_run;
    }
    shift = m_new == -INFINITY ? 0.f : m_new;
    alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - shift);
    return m_new;
  }

  // fp32 kernels: the online-softmax step on the tile's scores (reference point, denominator,
  // weights).  Returns alpha, the factor O^T must be multiplied by.
  //
  // MODE 0 and 1 first compute the weights against the current m.  When every lane's partial
  // denominator stays below 2^kLazy and no m is -inf, every weight is below 2^kLazy, so every
  // x - m is below kLazy (exp2 is monotonic and exact at 2^kLazy) and the rule keeps m: those
  // weights are the tile's, and the row maximum is never taken.  Otherwise the maximum decides,
  // and the weights are recomputed for the rows whose m moved.  Both ways give the same bits.
  // MODE 2-4 take the maximum first: under ALiBi the reference point of many rows moves at
  // every tile.
  __device__ __forceinline__ float weights(const Params &p, const f32x16 (&sc)[2]) { return weights(p, sc, pw); }
  __device__ __forceinline__ float weights(const Params &p, const f32x16 (&sc)[2], float (&wout)[2][16]) {
    if constexpr (MODE < 2) return weights_rest(p, sc, expw(p, sc, m_run == -INFINITY ? 0.f : m_run, wout), wout);
    float shift, alpha;
    const float m_new = ref_point(p, sc, shift, alpha);
    const float lsum = expw(p, sc, shift, wout);
    l_run = __builtin_fmaf(alpha, l_run, lsum);
    m_run = m_new;
    return alpha;
  }
  // MODE 0 and 1: weights() once the weights against the current m (and their sum lsum) are
  // in wout.
  __device__ __forceinline__ float weights_rest(const Params &p, const f32x16 (&sc)[2], float lsum,
                                                float (&wout)[2][16]) {
    static_assert(MODE < 2, "lazy reference point");
    if (!__ballot(m_run == -INFINITY || !(lsum < kLazyW))) {
      l_run = __builtin_fmaf(1.f, l_run, lsum);
      return 1.f;
    }
    float shift, alpha;
    const float m_new = ref_point(p, sc, shift, alpha);
    if (__ballot(m_new != m_run)) lsum = expw(p, sc, shift, wout);
    l_run = __builtin_fmaf(alpha, l_run, lsum);
    m_run = m_new;
    return alpha;
  }

  // O^T *= alpha (skipped when alpha == 1 in every lane: multiplying by 1 is exact)
  __device__ __forceinline__ void rescale(float alpha) {
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NOB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
  }

  // fp32 kernels: the whole online-softmax step of tile t on `sacc`, then pv().
  __device__ __forceinline__ void softmax(const Params &p, int t) {
    scores(p, t, sacc);
    if (!full(t)) select(t, sacc);
    rescale(weights(p, sacc));
  }

  // bf16 kernels: the online-softmax step of tile t on `sacc` and O^T = alpha O^T + V^T P^T
  // with the tile's V in `vl`, fused per 16-key chunk.  The reference point comes first (the
  // row maximum, every tile); then chunk c's weights, their bf16 rounding and partial sums, and
  // chunk c's PV MFMAs, whose execution overlaps the vector work of chunk c + 1.  The MFMAs are
  // ordered key chunk outer, d block inner, so that consecutive MFMAs accumulate into different
  // registers.
  __device__ __forceinline__ void softmax_pv(const Params &p, int t, const unsigned char *vl) {
    static_assert(DP == 1, "bf16 kernels own the whole d range");
    scores(p, t, sacc);
    if (!full(t)) select(t, sacc);
    float shift, alpha;
    const float m_new = ref_point(p, sacc, shift, alpha);
    rescale(alpha);
    {
      // The V^T operand of MFMA c comes from two transposing reads: within each 16-lane group,
      // lane r reads 4 d of key 16c + 8e + 4h + r/4, and lane i receives keys ... + j
      // (j = 0..3) at one d.
      const int r16 = lane & 15, dh = (lane >> 4) & 1;
      const int key_l = 4 * half + (r16 >> 2);  // key offset of this lane's read
      const int d_l = 16 * dh + 4 * (r16 & 3);  // d offset (elements) of this lane's read
      const uint32_t vbase_l = lds_addr(vl) + key_l * (D * 2) + (d_l & 7) * 2;
      // the swizzle depends on key % 4 (d = 128) or (key / 2) % 2 (d = 64), i.e. on key_l only
      uint32_t a0[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) a0[db] = vbase_l + ((((db * 32 + d_l) >> 3) ^ L::vsw(key_l)) * 16);
      s16x4 r[2][8];  // r[c & 1][2 db + e]: keys 16c + 8e + key_l of d block db
      auto issue = [&](int c) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          r[c & 1][2 * db] = read_v(a0[db], c, 0);
          r[c & 1][2 * db + 1] = read_v(a0[db], c, 1);
        }
      };
      // The denominator sums the weights as rounded for the PV product, so that o is a weighted
      // mean of the values with weights summing to one (a row that sees one key gets that key's
      // value exactly): pairs of bf16 weights by dot products with (1, 1), one chain per chunk,
      // the chains added in a fixed order.  (Each chain starts with the three-operand form and
      // an inline 0 addend, written out: the compiler would otherwise zero a register for the
      // accumulating two-operand form.)
      const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
      float acc[4];
      issue(0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // chunk c covers keys 16c..16c+15; lane half h supplies keys 16c + 8(j/4) + 4h + j%4,
        // which are its S^T registers i = 8(c%2) + j of block c/2
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = sacc[c >> 1][8 * (c & 1) + j];
          float w;
          if constexpr (MODE <= 1) w = __builtin_amdgcn_exp2f(__builtin_fmaf(x, p.scale_log2, -shift));
          else w = __builtin_amdgcn_exp2f(x - shift);
          pb[c][j] = (__bf16)w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x2 pr = {pb[c][2 * j], pb[c][2 * j + 1]};
          if (j == 0) asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(acc[c]) : "v"(pr), "v"(one));
          else acc[c] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc[c], false);
        }
        s16x4 *rc = r[c & 1];
        if (c + 1 < 4) {  // the reads for key block c + 1 are in flight during the MFMAs of c
          issue(c + 1);
          if constexpr (NDB == 4) lds_wait<8>(rc[0], rc[1], rc[2], rc[3], rc[4], rc[5], rc[6], rc[7]);
          else lds_wait<4>(rc[0], rc[1], rc[2], rc[3]);
        } else {
          if constexpr (NDB == 4) lds_wait<0>(rc[0], rc[1], rc[2], rc[3], rc[4], rc[5], rc[6], rc[7]);
          else lds_wait<0>(rc[0], rc[1], rc[2], rc[3]);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const s16x8 both = __builtin_shufflevector(rc[2 * db], rc[2 * db + 1], 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pb[c],
                                                             oacc[db], 0, 0, 0);
        }
      }
      l_run = __builtin_fmaf(alpha, l_run, (acc[0] + acc[1]) + (acc[2] + acc[3]));
      m_run = m_new;
    }
  }

  // fp32 kernels: O^T += V^T P^T with the tile's V in `vl`.  MFMA (kb, i) contracts 2 keys:
  // lane half h supplies key 32kb + 8(i/4) + 4h + i%4.
  __device__ __forceinline__ void pv(const unsigned char *vl) { pv(vl, pw); }
  __device__ __forceinline__ void pv(const unsigned char *vl, const float (&win)[2][16]) {
    static_assert(!BF16, "bf16 kernels take softmax_pv");
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
#pragma unroll
        for (int db = 0; db < NOB; ++db) {
          const int d = (dpart * NOB + db) * 32 + lq;
          const int ch = (d >> 2) ^ L::vsw(key);
          const float a = *reinterpret_cast<const float *>(vl + key * (D * 4) + ch * 16 + (d & 3) * 4);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, win[kb][i], oacc[db], 0, 0, 0);
        }
      }
  }
  // fp32 MODE 0 and 1: PV of the previous tile (V in `vl`, its weights `win`) and the weights of
  // the current tile's scores `sc` against the current m (the first step of weights(), into
  // `wout`), in one stretch of code so that the vector work runs beside the MFMAs.  Returns the
  // weights' partial sum, for weights_rest().
  __device__ __forceinline__ float pv_expw(const Params &p, const unsigned char *vl, const float (&win)[2][16],
                                           const f32x16 (&sc)[2], float (&wout)[2][16]) {
    static_assert(!BF16 && MODE < 2, "fp32, lazy reference point");
    const float shift = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
#pragma unroll
        for (int db = 0; db < NOB; ++db) {
          const int d = (dpart * NOB + db) * 32 + lq;
          const int ch = (d >> 2) ^ L::vsw(key);
          const float a = *reinterpret_cast<const float *>(vl + key * (D * 4) + ch * 16 + (d & 3) * 4);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, win[kb][i], oacc[db], 0, 0, 0);
        }
        wout[kb][i] = expw_one(p, sc[kb][i], shift);
      }
    return wsum(wout);
  }
  // transposing read of keys 16c + 8e + key_l (immediate offset), see softmax_pv()
  __device__ __forceinline__ static s16x4 read_v(uint32_t a, int c, int e) {
    switch (2 * c + e) {
      case 0: return lds_read_tr16<0 * D * 2>(a);
      case 1: return lds_read_tr16<8 * D * 2>(a);
      case 2: return lds_read_tr16<16 * D * 2>(a);
      case 3: return lds_read_tr16<24 * D * 2>(a);
      case 4: return lds_read_tr16<32 * D * 2>(a);
      case 5: return lds_read_tr16<40 * D * 2>(a);
      case 6: return lds_read_tr16<48 * D * 2>(a);
      default: return lds_read_tr16<56 * D * 2>(a);
    }
  }

  // bf16, d 128, no split: finish()'s values, stored through this wave's 8 KiB of LDS at `epi`
  // so that each global store writes four whole rows (16 bytes per lane) instead of 8 bytes per
  // lane across 32 rows.  Row r's 16-byte chunk c sits at r * 256 + (c ^ (r % 16)) * 16 there.
  __device__ __forceinline__ void finish_lds(const Params &p, int b, int head, int row0_wave, unsigned char *epi) {
    static_assert(BF16 && D == 128 && DP == 1, "bf16 rows of 256 bytes");
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float r4[4];
        // (+ 0 as in finish())
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = oacc[db][4 * g + e] * inv + 0.f;
        const u32x2 pk = {pack_bf16x2(r4[0], r4[1]), pack_bf16x2(r4[2], r4[3])};
        // registers 4g..4g+3 hold d 32 db + 8 g + 4 half ..: bytes 8 half.. of chunk 4 db + g
        const int c = 4 * db + g;
        *reinterpret_cast<u32x2 *>(epi + lq * 256 + ((c ^ (lq & 15)) * 16) + 8 * half) = pk;
      }
    unsigned char *obase = static_cast<unsigned char *>(p.o) +
                           ((int64_t)b * p.so_b + (int64_t)head * p.so_h + (p.q_start + row0_wave) * p.so_t) * ES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // rows 4 i .. 4 i + 3, lane l: row 4 i + l / 16, chunk l % 16
      const int r = 4 * i + (lane >> 4), c = lane & 15;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(epi + r * 256 + ((c ^ (r & 15)) * 16));
      if (row0_wave + r < p.Tq) *reinterpret_cast<u32x4 *>(obase + (int64_t)r * p.so_t * ES + c * 16) = v;
    }
    if (row_ok && p.lse && half == 0)
      p.lse[(int64_t)b * p.sl_b + (int64_t)head * p.sl_h + p.q_start + row] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }

  // o = a / l, lse = m + ln l; a row that saw nothing gets 0 and -inf.
  __device__ __forceinline__ void finish(const Params &p, int b, int head, int split) {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!row_ok) return;
    if (p.n_splits > 0) {
      const SplitSpan span(p.q_offset + row, p);
      if (span.single) {
        if (split != span.s_lo) return;  // nothing of this row here; its split writes o and lse
      } else {  // split-KV: the row's state goes to the workspace as it stands, for the merge
      const int64_t r = ((int64_t)split * p.B * p.Hq + (int64_t)b * p.Hq + head) * p.Tq_all + row;
      float *arow = p.ws_acc + r * D;
#pragma unroll
      for (int db = 0; db < NOB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v4 = {oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
          *reinterpret_cast<f32x4 *>(arow + (dpart * NOB + db) * 32 + 8 * g + 4 * half) = v4;
        }
      if (half == 0 && dpart == 0) {
        const f32x2 ml = {m_run, l_tot};
        *reinterpret_cast<f32x2 *>(p.ws_ml + 2 * r) = ml;
      }
      return;
      }
    }
    unsigned char *orow = static_cast<unsigned char *>(p.o) +
                          ((int64_t)b * p.so_b + (int64_t)head * p.so_h + (p.q_start + row) * p.so_t) * ES;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < NOB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = (dpart * NOB + db) * 32 + 8 * g + 4 * half;  // registers 4g..4g+3 hold d0..d0+3
        float r4[4];
        // (+ 0: a zero output is +0 whichever way it was reached, e.g. through a rescale by 0 of a
        // negative accumulator, so that a row's bits never depend on which tiles its wave processed)
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = oacc[db][4 * g + e] * inv + 0.f;
        if constexpr (BF16) {
          u32x2 pk = {pack_bf16x2(r4[0], r4[1]), pack_bf16x2(r4[2], r4[3])};
          *reinterpret_cast<u32x2 *>(orow + d0 * 2) = pk;
        } else {
          f32x4 v4 = {r4[0], r4[1], r4[2], r4[3]};
          *reinterpret_cast<f32x4 *>(orow + d0 * 4) = v4;
        }
      }
    if (p.lse && half == 0 && dpart == 0)
      p.lse[(int64_t)b * p.sl_b + (int64_t)head * p.sl_h + p.q_start + row] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
};

// ---------------------------------------------------------------------------------------
// The tile copy HBM -> LDS, split over the NW waves of the workgroup, as buffer loads that
// write LDS directly (buffer_load_dwordx4 ... lds: lane l of a wave writes bytes
// [16 l, 16 l + 16) of a 1 KiB LDS block).  The buffer resource covers the tile and the rest
// of the (b, KV head) slice; lane l copies row (blk * RB + l / CH), stored chunk l % CH, of its
// blocks at a fixed 32-bit offset.  Reads past the end of the slice (rows past Tk) return
// zeros.  The host checks that a slice spans less than 2 GiB.
// ---------------------------------------------------------------------------------------
template <bool BF16, int D, int NW>
struct Copier {
  using L = Layout<BF16, D>;
  static constexpr int ES = L::ES;
  static constexpr int BPW = L::NBLK / NW;  // 1 KiB blocks each wave copies per tensor per tile
  static_assert(L::NBLK % NW == 0, "blocks per tile must split evenly over the waves");
  const unsigned char *kbase, *vbase;  // the (b, KV head) slice, or the KV head in block 0 (paged)
  int64_t kbytes, vbytes;  // bytes of each slice from its first key to the end of key Tk - 1
  const int32_t *bt_row;   // paged: the block-table row of sequence b
  BufRsrc kslice, vslice;  // contiguous: the slices, from their first key to the end of key Tk - 1
  uint32_t kstep, vstep;   // contiguous: bytes from one tile of a slice to the next
  int wid;
  uint32_t koff[BPW], voff[BPW];

  __device__ __forceinline__ void init(const Params &p, int b, int kvh, int wid_, int lane) {
    wid = wid_;
    const int64_t bk = p.block_table ? 0 : b;
    bt_row = p.block_table ? p.block_table + (int64_t)b * p.bt_stride : nullptr;
    kbase = static_cast<const unsigned char *>(p.k) + (bk * p.sk_b + (int64_t)kvh * p.sk_h + p.k_start * p.sk_t) * ES;
    vbase = static_cast<const unsigned char *>(p.v) + (bk * p.sv_b + (int64_t)kvh * p.sv_h + p.k_start * p.sv_t) * ES;
    kbytes = ((int64_t)(p.Tk - 1) * p.sk_t + D) * ES;
    vbytes = ((int64_t)(p.Tk - 1) * p.sv_t + D) * ES;
    kslice = make_rsrc(kbase, kbytes);
    vslice = make_rsrc(vbase, vbytes);
    kstep = (uint32_t)(kBc * p.sk_t * ES);
    vstep = (uint32_t)(kBc * p.sv_t * ES);
    const int cp_row = lane / L::CH, cp_chunk = lane % L::CH;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int r = (wid * BPW + i) * L::RB + cp_row;
      koff[i] = (uint32_t)(r * p.sk_t * ES) + ((cp_chunk ^ L::ksw(r)) * 16);
      voff[i] = (uint32_t)(r * p.sv_t * ES) + ((cp_chunk ^ L::vsw(r)) * 16);
    }
  }
  // Paged: the resource of tile t of K (IS_K) or V, the tile's rows in its block; rows past
  // the sequence's keys, and a block index outside [0, num_blocks), read as zeros.
  template <bool IS_K>
  __device__ __forceinline__ BufRsrc paged_rsrc(const Params &p, int t) const {
    const int64_t sb = IS_K ? p.sk_b : p.sv_b, st = IS_K ? p.sk_t : p.sv_t;
    const uint32_t key0 = (uint32_t)t * kBc;  // < Tk < 2^31
    const int64_t rows = min((int64_t)kBc, (int64_t)p.Tk - key0);
    const int32_t blk = rows > 0 ? load_const(bt_row + key0 / (uint32_t)p.block_size) : -1;
    const bool ok = blk >= 0 && blk < p.num_blocks;
    const int64_t in_blk = key0 % (uint32_t)p.block_size;
    return make_rsrc((IS_K ? kbase : vbase) + ((ok ? blk : 0) * sb + in_blk * st) * ES,
                     ok ? ((rows - 1) * st + D) * ES : 0);
  }
  // Where the copies of tile t of K (IS_K) or V read: a resource and a byte offset added to
  // each lane's.  Contiguous: the slice and the tile's place in it (rows past Tk lie past the
  // slice's end and read zeros; the host keeps a slice under 2 GiB, so the offsets fit 32
  // bits); paged: the tile's own resource.
  // `inside`: a contiguous tile wholly inside the keys, which global loads may read.
  struct Src {
    BufRsrc rs;
    uint32_t add;
    bool inside;
    const unsigned char *base;  // contiguous: the slice's first key
  };
  template <bool IS_K>
  __device__ __forceinline__ Src src(const Params &p, int t) const {
    if (bt_row) return Src{paged_rsrc<IS_K>(p, t), 0u, false, IS_K ? kbase : vbase};
    return Src{IS_K ? kslice : vslice, (uint32_t)t * (IS_K ? kstep : vstep), (int64_t)t * kBc + kBc <= p.Tk,
               IS_K ? kbase : vbase};
  }
  // Contiguous keys only: point at the slice of (b, kvh) (the lane offsets stay).
  __device__ __forceinline__ void rebase(const Params &p, int b, int kvh) {
    kbase = static_cast<const unsigned char *>(p.k) + ((int64_t)b * p.sk_b + (int64_t)kvh * p.sk_h) * ES;
    vbase = static_cast<const unsigned char *>(p.v) + ((int64_t)b * p.sv_b + (int64_t)kvh * p.sv_h) * ES;
    kslice = make_rsrc(kbase, kbytes);
    vslice = make_rsrc(vbase, vbytes);
  }
  // This wave's byte offset into a tile's LDS buffer.  Passed through an empty asm statement
  // where a tile's copies are issued, so that the compiler forms each copy's LDS address
  // (a scalar add) there instead of keeping all of them live in SGPRs across the tile loop,
  // which runs out of SGPRs and spills them to VGPR lanes (a v_readlane per copy).
  __device__ __forceinline__ uint32_t wave_off() const {
    uint32_t w = (uint32_t)(wid * BPW * 1024);
    asm volatile("" : "+s"(w));
    return w;
  }
  // K copy i (of BPW) and V copy i of a tile from its sources into the LDS buffer at kdst / vdst
  // (wo = wave_off()); GLB: by global loads from the tile's base address (the tile must be
  // `inside`), else through the buffer resource.
  template <bool GLB>
  __device__ __forceinline__ void copy_k(const Src &s, int i, unsigned char *kdst, uint32_t wo) const {
    if constexpr (GLB) glb_load_lds16(s.base + s.add, kdst + wo + i * 1024, koff[i]);
    else buf_load_lds16(s.rs, kdst + wo + i * 1024, koff[i] + s.add);
  }
  template <bool GLB>
  __device__ __forceinline__ void copy_v(const Src &s, int i, unsigned char *vdst, uint32_t wo) const {
    if constexpr (GLB) glb_load_lds16(s.base + s.add, vdst + wo + i * 1024, voff[i]);
    else buf_load_lds16(s.rs, vdst + wo + i * 1024, voff[i] + s.add);
  }
  __device__ __forceinline__ void tiles(const Params &p, int t, unsigned char *kdst, unsigned char *vdst) const {
    const Src ks = src<true>(p, t), vs = src<false>(p, t);
    const uint32_t wo = wave_off();
#pragma unroll
    for (int i = 0; i < BPW; ++i) copy_k<false>(ks, i, kdst, wo);
#pragma unroll
    for (int i = 0; i < BPW; ++i) copy_v<false>(vs, i, vdst, wo);
  }
};

// ---------------------------------------------------------------------------------------
// Mask tiles through LDS (MODE 1 when the workgroup's MR rows share their mask rows across its
// heads, mask rows contiguous and 16-byte aligned): the MR x 64 fp32 block of tile t, each
// entry divided by the scale (fl(mask * fl(1 / scale)), the value mask_acc() starts the score
// accumulators at), row-major 256 bytes per row with the 16-byte chunks of row r stored at
// chunk ^ (r % 16).  The waves load the next tile's block into registers one tile ahead (MR / 4
// blocks of 4 rows, split over the waves), divide it and write it to LDS at the end of the
// step, so the division is done once per workgroup rather than once per head.  MR is 64 for
// 8-wave workgroups (two 32-row halves of 4 heads each), else 32.  Rows past Tq and entries
// past the mask's last valid entry read as zeros; other entries past Tk belong to keys that
// the select removes.
// ---------------------------------------------------------------------------------------
template <int NW>
struct MaskStager {
  static constexpr int MR = NW == 8 ? 64 : 32;  // staged rows
  static constexpr int MPW = MR / 4 / NW;       // 1 KiB blocks each wave stages per tile
  const unsigned char *base;          // mask row row0 of the workgroup, key 0
  int64_t bytes_to_end;               // from base to the end of entry (Tq - 1, Tk - 1)
  uint32_t off[MPW], lds_off[MPW];
  __device__ __forceinline__ void init(const Params &p, int b, int row0, int wid, int lane) {
    base = reinterpret_cast<const unsigned char *>(p.mask + (int64_t)b * p.sm_b + (int64_t)row0 * p.sm_i);
    bytes_to_end = ((int64_t)(p.Tq - 1 - row0) * p.sm_i + p.Tk) * 4;
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      // lane l of block k holds stored chunk l % 16 of row 4 k + l / 16, i.e. logical chunk
      // (l % 16) ^ (row % 16)
      const int r = (wid * MPW + i) * 4 + lane / 16;
      const uint32_t c = (uint32_t)(lane % 16) ^ (uint32_t)(r & 15);
      off[i] = (uint32_t)(r * p.sm_i * 4) + c * 16u;
      lds_off[i] = (uint32_t)((wid * MPW + i) * 1024 + lane * 16);
    }
  }
  __device__ __forceinline__ BufRsrc rsrc(int t) const {
    const int64_t skip = (int64_t)t * kBc * 4;
    return make_rsrc(base + skip, bytes_to_end - skip);
  }
  __device__ __forceinline__ void load(BufRsrc rs, u32x4 (&v)[MPW]) const {
#pragma unroll
    for (int i = 0; i < MPW; ++i) v[i] = buf_load16(rs, off[i]);
  }
  __device__ __forceinline__ void store(const Params &p, const u32x4 (&v)[MPW], unsigned char *dst) const {
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      f32x4 m4;
#pragma unroll
      for (int e = 0; e < 4; ++e) m4[e] = __uint_as_float(v[i][e]) * p.inv_scale;
      *reinterpret_cast<f32x4 *>(dst + lds_off[i]) = m4;
    }
  }
};

// ---------------------------------------------------------------------------------------
// Streaming kernel (1, 2, 4 or 8 waves): each wave walks the tiles; the next tile is copied into
// the other pair of LDS buffers while the current one is used, its copies spread over the QK
// steps of the current tile.
// ---------------------------------------------------------------------------------------
// bf16 kernels are built for 2 waves per SIMD; fp32 ones (matrix-bound, larger tiles) and the
// general score-variant kernel (MODE 2, whose extra registers would spill at 2) for 1, except
// 8-wave workgroups, which put 2 waves on each SIMD by construction.  The mask-free variant
// kernels (MODE 3, 4) take 2: MODE 3 spills a few registers there and still runs ≈ 10 % faster
// than at 1, MODE 4 ≈ 25 %.
template <bool BF16, int D, int NW, int MODE, int DP = 1, bool PERS = false>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(MODE == 2 ? (NW == 8 ? 2 : 1) : (BF16 || NW == 8) ? 2 : 1)))
fa_fwd_kernel(Params p0) {
  using L = Layout<BF16, D>;
  using CP = Copier<BF16, D, NW>;
  constexpr int NDS = D / 16;        // QK steps of a tile
  constexpr int NCP = 2 * CP::BPW;   // copies of a tile per wave
  // four LDS buffers as four objects, so that the compiler can tell the copies into one from
  // the reads of another and does not wait for the copies before those reads
  __shared__ __attribute__((aligned(1024))) unsigned char k0[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[L::TILE_BYTES];
  constexpr int MBYTES = MODE == 1 ? MaskStager<NW>::MR * 256 : 16;  // staged mask blocks (MODE 1)
  __shared__ __attribute__((aligned(1024))) unsigned char m0[MBYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char m1[MBYTES];
  // PERS: each wave's output rows on their way to HBM (Wave::finish_lds)
  __shared__ __attribute__((aligned(1024))) unsigned char epi[PERS ? NW * 8192 : 16];

  // the wave index is uniform: keep it (and the LDS addresses derived from it) in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  // PERS (persistent launch, one workgroup per CU, contiguous keys, no split or per-sequence
  // lengths): workgroup g walks the launch indices x + 8 idx that a one-item-per-workgroup
  // launch would send to its XCD x = g % 8, idx = k nW + (j or nW - 1 - j) for its k-th item
  // (j = g / 8, nW = workgroups per XCD): a snake over the XCD's items, which balances causal
  // work when the items come heaviest first.
  auto item_of = [&](int k) -> int {
    const int g = (int)blockIdx.x, x = g & 7, j = g >> 3, nW = (int)(gridDim.x >> 3);
    const int cx = (p0.n_blocks - x + 7) >> 3;  // launch indices below n_blocks on XCD x
    const int idx = k * nW + ((k & 1) ? nW - 1 - j : j);
    return idx < cx ? x + 8 * idx : -1;
  };
  Work wk(p0, PERS ? item_of(0) : (int)blockIdx.x);
  const Params p = seq_params(p0, wk.b);
  wk.set_range(p);
  // split-KV: no row of this work item sees a key of its split, so the merge reads none of its
  // states (split 0 keeps the sink term and always writes them)
  if (p.n_splits > 0 && wk.t_begin >= wk.t_end && (wk.split != 0 || p.sinks == nullptr)) return;
  const int G = p.heads_per_block;
  // wave wid: part wid % DP of the d range, head wq % G, rows (wq / G) * 32 of the block
  const int wq = wid / DP;
  int head = wk.head_base + wq % G;
  Wave<BF16, D, MODE, DP> wv;
  wv.init(p, wk.b, head, wk.row0_blk + (wq / G) * kRowsWave, lane, wk.split == 0, wid % DP);
  CP cp;
  cp.init(p, wk.b, wk.kvh, wid, lane);
  using MS = MaskStager<NW>;
  MS ms;
  const bool mlds = MODE == 1 && p.mask_lds;
  if (mlds) {
    ms.init(p, wk.b, wk.row0_blk, wid, lane);
    wv.mask_lds_row = (uint32_t)((wq / G) * kRowsWave + (lane & 31));
  }


  // GLB: the next tile's copies by global loads (every tile the work item copies lies wholly
  // inside contiguous keys), else through the buffer resources.  Chosen once per work item, so
  // that neither a copy nor a step carries a branch of its own.
  auto step = [&](auto glb, int t, const unsigned char *kc, const unsigned char *vc, const unsigned char *mcur,
                  unsigned char *kn, unsigned char *vn, unsigned char *mnext) __attribute__((always_inline)) {
    constexpr bool GLB = decltype(glb)::value;
    const bool has_next = t + 1 < wk.t_end;  // the buffers kn, vn were released by the last barrier
    if constexpr (GLB) {
      // The lanes' copy offsets pass through empty asm statements once per tile, so that the
      // compiler cannot hoist their 64-bit forms out of the loop: each global copy then takes
      // the tile's base address from SGPRs and the 32-bit lane offset as is (no vector add).
#pragma unroll
      for (int i = 0; i < CP::BPW; ++i) {
        asm("" : "+v"(cp.koff[i]));
        asm("" : "+v"(cp.voff[i]));
      }
    }
    const typename CP::Src ks = cp.template src<true>(p, t + 1), vs = cp.template src<false>(p, t + 1);
    // MODE 1 with a staged mask: this wave's share of the next tile's block, loaded now and
    // written to LDS (divided by the scale) at the end of the step
    u32x4 mnv[MS::MPW];
    if (mlds && has_next) ms.load(ms.rsrc(t + 1), mnv);
    auto copies = [&](int ds) {  // copy i goes with QK step i * NDS / NCP
      if (has_next) {
        const uint32_t wo = cp.wave_off();
#pragma unroll
        for (int i = 0; i < NCP; ++i)
          if (i * NDS / NCP == ds) {
            if (i < CP::BPW) cp.template copy_k<GLB>(ks, i, kn, wo);
            else cp.template copy_v<GLB>(vs, i - CP::BPW, vn, wo);
          }
      }
    };
    if (wv.active(t)) {
      if constexpr (MODE == 1) wv.mask_acc(p, t, mcur, wv.sacc);
      wv.template qk<true>(kc, wv.sacc, copies);
      if constexpr (BF16) {
        wv.softmax_pv(p, t, vc);
      } else {
        wv.softmax(p, t);
        wv.pv(vc);
      }
    } else {
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) copies(ds);
    }
    if (mlds && has_next) ms.store(p, mnv, mnext);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of tile t + 1 have landed
    __syncthreads();                // ... everyone's have, and buffers kc, vc are free again
  };
  if constexpr (PERS) {
    // every work item in turn, each as a one-item workgroup would take it (every tile lies
    // inside the keys: checked by the host)
    static_assert(MODE != 1, "no staged mask in the persistent loop");
    for (int k = 1;; ++k) {
      if (wk.t_begin < wk.t_end) {
        cp.tiles(p, wk.t_begin, k0, v0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int t = wk.t_begin; t < wk.t_end; t += 2) {
          step(std::true_type{}, t, k0, v0, m0, k1, v1, m1);
          if (t + 1 < wk.t_end) step(std::true_type{}, t + 1, k1, v1, m1, k0, v0, m0);
        }
      }
      wv.finish_lds(p, wk.b, head, wk.row0_blk + (wq / G) * kRowsWave, epi + wid * 8192);
      const int vb = item_of(k);
      if (vb < 0) break;
      wk = Work(p0, vb);
      wk.set_range(p);
      head = wk.head_base + wq % G;
      wv.init(p, wk.b, head, wk.row0_blk + (wq / G) * kRowsWave, lane, true, wid % DP);
      cp.rebase(p, wk.b, wk.kvh);
    }
    return;
  }
  if (wk.t_begin < wk.t_end) {
    cp.tiles(p, wk.t_begin, k0, v0);
    if (mlds) {
      u32x4 mv[MS::MPW];
      ms.load(ms.rsrc(wk.t_begin), mv);
      ms.store(p, mv, m0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  auto run = [&](auto glb) __attribute__((always_inline)) {
    for (int t = wk.t_begin; t < wk.t_end; t += 2) {
      step(glb, t, k0, v0, m0, k1, v1, m1);
      if (t + 1 < wk.t_end) step(glb, t + 1, k1, v1, m1, k0, v0, m0);
    }
  };
  // (not for the additive mask, whose kernel has no registers to spare for a second loop)
  if (MODE != 1 && cp.template src<true>(p, wk.t_end - 1).inside) run(std::integral_constant<bool, MODE != 1>{});
  else run(std::false_type{});
  if constexpr (BF16 && D == 128 && DP == 1) {
    // the tile buffers are free after the last step's barrier: 8 KiB of them per wave
    if (p.n_splits == 0) {
      const int bi = (wid >> 1) & 3;
      unsigned char *buf = bi == 0 ? k0 : bi == 1 ? k1 : bi == 2 ? v0 : v1;
      wv.finish_lds(p, wk.b, head, wk.row0_blk + (wq / G) * kRowsWave, buf + (wid & 1) * 8192);
      return;
    }
  }
  wv.finish(p, wk.b, head, wk.split);
}

// ---------------------------------------------------------------------------------------
// fp32, one 32-row block of one head per workgroup of 4 waves with split roles.  An fp32 tile
// costs a wave 2 x (D / 2) MFMAs for the scores of its two 32-key blocks and 2 x D / 2 more for
// the PV product, one chain after the other, which makes a lone block's serial chain long.
// Here waves 0 and 1 compute the scores of key block 0 and 1 (Wave::qk_block: the chain of
// Wave::qk for that block) one tile ahead and hand them over through LDS, while waves 2 and 3
// keep the rows' online-softmax state and the output for their half of d (the arithmetic of
// the d-part waves, DP = 2).  A softmax wave issues the PV MFMAs of tile u - 1 and then takes
// the softmax step of tile u, whose vector work runs beside those MFMAs; the output sees the
// same operations in the same order (rescale for u - 1, PV of u - 1, rescale for u, ...), so
// every row gets the bits of the one-wave kernel.
//
// Step u (from t_begin - 1 to t_end; one barrier each): the score waves compute S(u + 1) from
// K(u + 1) and, between the MFMAs of that chain, copy K(u + 2) and V(u); the softmax waves
// issue PV(u - 1) from V(u - 1) and the weights of u - 1 together with tile u's weights against
// the current m (Wave::pv_expw), then finish the softmax step of u.  Tile t lives in K, V, S
// and weight buffers (t - t_begin) % 2, so a step writes only buffers that the step before it
// was the last to read.
// ---------------------------------------------------------------------------------------
constexpr int kSBytes = 2 * 16 * 64 * 4;  // S^T of one tile: [key block][register / 4][lane][4] fp32

template <int D>
__global__ void __launch_bounds__(320) fa_fwd_so_kernel(Params p0) {
  using L = Layout<false, D>;
  using CP = Copier<false, D, 1>;  // wave 4 copies the tiles
  __shared__ __attribute__((aligned(1024))) unsigned char k0[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char s0[kSBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char s1[kSBytes];

  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  Work wk(p0);
  const Params p = seq_params(p0, wk.b);
  wk.set_range(p);
  if (wk.t_begin >= wk.t_end) {  // no key for these rows: zeros and -inf
    if (wid == 2 || wid == 3) {
      Wave<false, D, 0, 2> wv;
      wv.init(p, wk.b, wk.head_base, wk.row0_blk, lane, true, wid - 2);
      wv.finish(p, wk.b, wk.head_base, 0);
    }
    return;
  }
  const int head = wk.head_base;  // one head per workgroup

  // The step schedule, one barrier per step, the same for every wave; each role runs it in a
  // loop of its own, so that no role's registers stay live through another's work.
  // body(u, kr, sw, sr, vr, wr, wn, kw, vw); j = u - t_begin + 1 even: tile u + 1 is in slot 0,
  // tiles u and u - 1 in slots 1 and 0.
  auto run = [&](auto &&body, float (&w0)[2][16], float (&w1)[2][16]) __attribute__((always_inline)) {
    for (int u = wk.t_begin - 1; u <= wk.t_end; u += 2) {
      body(u, k0, s0, s1, v0, w0, w1, k1, v1);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies and LDS writes are done
      __syncthreads();                // ... everyone's, and the buffers read in this step are free
      if (u + 1 <= wk.t_end) {
        body(u + 1, k1, s1, s0, v1, w1, w0, k0, v0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
  };

  if (wid == 4) {
    // copy wave: K(t_begin) first, then K(u + 2) and V(u) in step u
    CP cp;
    cp.init(p, wk.b, wk.kvh, 0, lane);
    {
      const typename CP::Src ks = cp.template src<true>(p, wk.t_begin);
      const uint32_t wo = cp.wave_off();
#pragma unroll
      for (int i = 0; i < CP::BPW; ++i) cp.template copy_k<false>(ks, i, k0, wo);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float wd[2][16];
    run([&](int u, const unsigned char *, unsigned char *, const unsigned char *, const unsigned char *,
            float (&)[2][16], float (&)[2][16], unsigned char *kw, unsigned char *vw) __attribute__((always_inline)) {
          // a tile wholly inside the keys by global loads (its base address in SGPRs, no vector
          // work per copy), else through the buffer resource.  The lane offsets pass through
          // empty asm statements, so that the compiler keeps them 32-bit (see fa_fwd_kernel).
#pragma unroll
          for (int i = 0; i < CP::BPW; ++i) {
            asm("" : "+v"(cp.koff[i]));
            asm("" : "+v"(cp.voff[i]));
          }
          const uint32_t wo = cp.wave_off();
          if (u + 2 < wk.t_end) {
            const typename CP::Src ks = cp.template src<true>(p, u + 2);
            if (ks.inside) {
#pragma unroll
              for (int i = 0; i < CP::BPW; ++i) cp.template copy_k<true>(ks, i, kw, wo);
            } else {
#pragma unroll
              for (int i = 0; i < CP::BPW; ++i) cp.template copy_k<false>(ks, i, kw, wo);
            }
          }
          if (u >= wk.t_begin && u < wk.t_end) {
            const typename CP::Src vs = cp.template src<false>(p, u);
            if (vs.inside) {
#pragma unroll
              for (int i = 0; i < CP::BPW; ++i) cp.template copy_v<true>(vs, i, vw, wo);
            } else {
#pragma unroll
              for (int i = 0; i < CP::BPW; ++i) cp.template copy_v<false>(vs, i, vw, wo);
            }
          }
        }, wd, wd);
    return;
  }
  if (wid < 2) {
    // score waves: S(u + 1) in step u
    Wave<false, D, 0, 2> wv;
    wv.init(p, wk.b, head, wk.row0_blk, lane, false);
    __syncthreads();  // K(t_begin) has landed
    float wd[2][16];
    run([&](int u, const unsigned char *kr, unsigned char *sw, const unsigned char *, const unsigned char *,
            float (&)[2][16], float (&)[2][16], unsigned char *, unsigned char *) __attribute__((always_inline)) {
          if (u + 1 < wk.t_end) {
            f32x16 sc;
            wv.qk_block(kr, wid, sc, [](int) {});
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 v4 = {sc[4 * g], sc[4 * g + 1], sc[4 * g + 2], sc[4 * g + 3]};
              *reinterpret_cast<f32x4 *>(sw + ((wid * 4 + g) * 64 + lane) * 16) = v4;
            }
          }
        }, wd, wd);
    return;
  }
  // softmax waves: PV(u - 1) and the softmax step of u in step u
  Wave<false, D, 0, 2> wv;
  wv.init(p, wk.b, head, wk.row0_blk, lane, true, wid - 2, false);
  __syncthreads();  // K(t_begin) has landed
  float w0[2][16], w1[2][16];  // the weights of the tiles in slot 0 and 1
  run([&](int u, const unsigned char *, unsigned char *, const unsigned char *sr, const unsigned char *vr,
          float (&wr)[2][16], float (&wn)[2][16], unsigned char *, unsigned char *) __attribute__((always_inline)) {
        const bool pv_due = u - 1 >= wk.t_begin, sm_due = u >= wk.t_begin && u < wk.t_end;
        if (sm_due) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 v4 = *reinterpret_cast<const f32x4 *>(sr + ((kb * 4 + g) * 64 + lane) * 16);
#pragma unroll
              for (int e = 0; e < 4; ++e) wv.sacc[kb][4 * g + e] = v4[e];
            }
          if (!wv.full(u)) wv.select(u, wv.sacc);
        }
        if (pv_due && sm_due) {
          const float lsum = wv.pv_expw(p, vr, wr, wv.sacc, wn);  // PV(u - 1) beside tile u's weights
          wv.rescale(wv.weights_rest(p, wv.sacc, lsum, wn));
        } else if (pv_due) {
          wv.pv(vr, wr);
        } else if (sm_due) {
          wv.rescale(wv.weights(p, wv.sacc, wn));
        }
      }, w0, w1);
  wv.finish(p, wk.b, head, 0);
}

// ---------------------------------------------------------------------------------------
// Split-KV merge ("FlashAttention forward in C", "Going further": the partial (m, l, a) of
// the key splits are combined with the same rescale as the tiles).  One wave per query row
// that sees more than one split, over the splits that meet the row's visible keys (and split 0
// with a sink; the states of other splits were never written):
//   M = max of m_s over the splits with l_s > 0
//   l = sum_s 2^(m_s - M) l_s,  a = sum_s 2^(m_s - M) a_s      (s ascending, fixed order)
//   o = l > 0 ? a * (1 / l) : 0,  lse = l > 0 ? (M + log2 l) ln 2 : -inf
// With one split this is the epilogue of the unsplit kernel, bit for bit.
// ---------------------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(256) void fa_merge_kernel(Params p0) {
  constexpr int EPL = D / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  // grid (ceil(Tq / 4), Hq, B): wave w of block x takes row 4 x + w of head y of sequence z
  const int64_t rows = (int64_t)p0.B * p0.Hq * p0.Tq_all;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6), h = blockIdx.y, b = blockIdx.z;
  if (i >= p0.Tq_all) return;
  const int64_t r = ((int64_t)b * p0.Hq + h) * p0.Tq_all + i;
  const Params p = seq_params(p0, b);
  if (i >= p.Tq) return;  // past the rows of a packed sequence
  const SplitSpan span(p.q_offset + i, p);
  if (span.single) return;  // finished by its split's work item
  const f32x2 *ml = reinterpret_cast<const f32x2 *>(p.ws_ml) + r;  // split s at ml[s * rows]

  // The splits read: those meeting the row's visible keys, and split 0 when it holds the sink
  // (the states of other splits were never written); the k-th, k < ns, in ascending order.
  int s_lo = span.s_lo, s_hi = span.s_hi;
  const bool with0 = p.sinks && s_lo > 0;
  if (p.sinks && s_hi == 0) s_hi = 1;
  const int ns = s_hi - s_lo + (with0 ? 1 : 0);
  auto split_of = [&](int k) { return with0 ? (k == 0 ? 0 : s_lo + k - 1) : s_lo + k; };
  auto bcast = [](float x, int k) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k)); };

  // M: lane k reads the k-th split's state (64 at a time); the maximum is exact in any order
  float M = -INFINITY;
  for (int k0 = 0; k0 < ns; k0 += 64) {
    float mk = -INFINITY;
    if (k0 + lane < ns) {
      const f32x2 st = ml[(int64_t)split_of(k0 + lane) * rows];
      if (st[1] > 0.f) mk = st[0];
    }
    const int n = min(64, ns - k0);
    for (int k = 0; k < n; ++k) M = fmaxf(M, bcast(mk, k));
  }

  // l and a summed over the splits in ascending order; split s has weight w_s = 2^(m_s - M),
  // 0 when it saw no key.  Lane k computes w_k; every lane takes the weights in order.
  float l = 0.f, a[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) a[e] = 0.f;
  for (int k0 = 0; k0 < ns; k0 += 64) {
    float w = 0.f, ls = 0.f;
    if (k0 + lane < ns) {
      const f32x2 st = ml[(int64_t)split_of(k0 + lane) * rows];
      if (st[1] > 0.f) { w = __builtin_amdgcn_exp2f(st[0] - M); ls = st[1]; }
    }
    const int n = min(64, ns - k0);
    for (int j0 = 0; j0 < n; j0 += 8) {  // 8 splits' accumulator loads in flight at a time
      float wj[8], lj[8], v[8][EPL];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        wj[j] = j0 + j < n ? bcast(w, j0 + j) : 0.f;
        lj[j] = j0 + j < n ? bcast(ls, j0 + j) : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (wj[j] > 0.f) {
          const float *as = p.ws_acc + ((int64_t)split_of(k0 + j0 + j) * rows + r) * D + EPL * lane;
#pragma unroll
          for (int e = 0; e < EPL; ++e) v[j][e] = as[e];
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) v[j][e] = 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (!(wj[j] > 0.f)) continue;  // splits that saw no key of this row add nothing
        l = l + wj[j] * lj[j];
#pragma unroll
        for (int e = 0; e < EPL; ++e) a[e] = a[e] + wj[j] * v[j][e];
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) a[e] = a[e] * inv + 0.f;  // as in Wave::finish: zeros are +0
  unsigned char *orow = static_cast<unsigned char *>(p.o) +
                        ((int64_t)b * p.so_b + (int64_t)h * p.so_h + (p.q_start + i) * p.so_t) * (BF16 ? 2 : 4);
  if constexpr (BF16) {
    if constexpr (EPL == 2)
      *reinterpret_cast<uint32_t *>(orow + 4 * lane) = pack_bf16x2(a[0], a[1]);
    else
      *reinterpret_cast<unsigned short *>(orow + 2 * lane) = __builtin_bit_cast(unsigned short, (__bf16)a[0]);
  } else {
    if constexpr (EPL == 2) {
      const f32x2 v = {a[0], a[1]};
      *reinterpret_cast<f32x2 *>(orow + 8 * lane) = v;
    } else {
      *reinterpret_cast<float *>(orow + 4 * lane) = a[0];
    }
  }
  if (p.lse && lane == 0)
    p.lse[(int64_t)b * p.sl_b + (int64_t)h * p.sl_h + p.q_start + i] = l > 0.f ? (M + log2f(l)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------------------
// Host side: validation (before any launch or write), geometry, dispatch.
// ---------------------------------------------------------------------------------------

typedef void (*KernelFn)(Params);

template <bool BF16, int D, int NW>
KernelFn pick_mode(int mode) {
  if constexpr (BF16 && NW >= 4) {
    if (mode == 3) return fa_fwd_kernel<BF16, D, NW, 3>;
    if (mode == 4) return fa_fwd_kernel<BF16, D, NW, 4>;
  }
  // elsewhere the general variant kernel serves modes 3 and 4 (same arithmetic)
  return mode >= 2 ? fa_fwd_kernel<BF16, D, NW, 2> : mode ? fa_fwd_kernel<BF16, D, NW, 1> : fa_fwd_kernel<BF16, D, NW, 0>;
}

template <bool BF16, int D>
KernelFn pick_nw(int nw, int mode) {
  switch (nw) {
    case 1: return pick_mode<BF16, D, 1>(mode);
    case 2: return pick_mode<BF16, D, 2>(mode);
    case 8: return pick_mode<BF16, D, 8>(mode);
    default: return pick_mode<BF16, D, 4>(mode);
  }
}

bool aligned(const void *ptr, int64_t a) { return (reinterpret_cast<uintptr_t>(ptr) % (uintptr_t)a) == 0; }

// Compute units of the current device (0 if unknown), looked up once per device.
int cu_count() {
  constexpr int kDevs = 64;
  static std::mutex mu;
  static int cache[kDevs] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// Picks (rows_per_block, heads_per_block): 4 waves with as many heads of one KV group as
// divide the group, falling back to fewer waves per workgroup only when 4-wave workgroups
// would leave some of the 256 CUs without one (at one workgroup per CU, 4 waves sharing each
// staged tile beat twice as many 2-wave workgroups: ≈ 20 % on a 2,044-token, 16-head causal
// prefill).  `eight`: the plain bf16 d = 128 kernel, whose 8-wave workgroups (one per CU, two
// waves per SIMD) measure ≈ 1 % faster than two 4-wave ones when there are at least two
// rounds of them.  Any choice gives the same bits.
void auto_tiling(int64_t B, int64_t Hkv, int64_t group, int64_t Tq, bool eight, int32_t *rows, int32_t *heads) {
  for (int nw = eight ? 8 : 4; nw >= 1; nw /= 2) {
    int g = 1;
    for (int c = nw; c >= 2; c /= 2)
      if (group % c == 0) { g = c; break; }
    const int64_t r = 32 * nw / g;
    const int64_t blocks = B * Hkv * (group / g) * ((Tq + r - 1) / r);
    if (blocks >= (nw == 8 ? 512 : 256) || nw == 1) {
      *heads = g;
      *rows = (int32_t)r;
      return;
    }
  }
}

// The key tiles a block of query rows [r0, r1) walks: the union of its rows' visible keys, as
// Work::set_range counts them.
int64_t block_tiles(int64_t r0, int64_t r1, int64_t q_offset, int64_t Tk, int causal, int64_t window) {
  const int64_t hi = causal ? std::min(q_offset + r1, Tk) : Tk;
  const int64_t lo = window > 0 ? std::max((int64_t)0, q_offset + r0 - window + 1) : 0;
  return hi > lo ? (hi + 63) / 64 - lo / 64 : 0;
}

// fp32 with plain scores: whether the split-role kernel (32-row one-head blocks on five waves,
// each tile's MFMA chain split over them: ≈ 1/3 of a 4-wave workgroup's time per tile, for 1/4
// of its rows) beats the auto geometry (rows, heads).  It does where the longest item's chain of
// tiles outweighs the total work: where the work of the auto geometry, at one workgroup per CU,
// takes fewer rounds than 3/4 of that chain (a 2,044-token causal prefill at 16/8 heads: 25 %
// faster; 4,096 tokens, or no causal mask: 13-17 % slower).  Any choice gives the same bits.
bool prefer_split_role(int64_t B, int64_t Hkv, int64_t group, int64_t Tq, int64_t Tk, int32_t rows, int32_t heads,
                       int64_t q_offset, int causal, int64_t window, int ncu) {
  const int64_t n_rt = (Tq + rows - 1) / rows;
  if (ncu <= 0 || rows * heads <= 32 || n_rt > 4096) return false;
  int64_t sum = 0, longest = 0;
  for (int64_t rt = 0; rt < n_rt; ++rt) {
    const int64_t t = block_tiles(rt * rows, std::min(Tq, (rt + 1) * rows), q_offset, Tk, causal, window);
    sum += t;
    longest = std::max(longest, t);
  }
  // (in double: the product can pass 2^63 for sizes the launch itself later refuses)
  const double total = (double)sum * (double)B * (double)Hkv * (double)(group / heads);
  return longest > 0 && 4.0 * total < 3.0 * (double)longest * ncu;
}

// Geometry of a split-KV call: the splits supply the parallelism, so a workgroup takes as many
// heads of one KV group as divide it (up to 4, sharing each staged K/V tile) and at most 4
// waves; a decode row (Tq = 1) then costs one wave per head.
void split_tiling(int64_t group, int64_t Tq, int32_t *rows, int32_t *heads) {
  const int g = group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
  int nw = g;
  while (nw < 4 && (int64_t)32 * nw / g < Tq) nw *= 2;
  *heads = g;
  *rows = 32 * nw / g;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split size (keys, a multiple of 64) for fa_fwd_splitkv when the caller has none: enough
// splits over the keys some row can see that the work items fill a 256-CU part twice, with at
// least 4 tiles per split for bf16 and 2 for fp32 (whose tiles cost more arithmetic).  A
// function of the arguments only, so results do not depend on the device.
int64_t default_split_keys(int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk,
                           int64_t q_offset, int causal, int64_t window, fa_dtype dtype) {
  if (Hkv <= 0 || Tq <= 0 || Tk <= 0 || B <= 0) return 64;
  const int64_t group = Hq / Hkv;
  int32_t rows = 0, heads = 0;
  split_tiling(group, Tq, &rows, &heads);
  const int64_t base = B * Hkv * (group / heads) * ceil_div(Tq, rows);
  const int64_t hi = causal ? std::min(Tk, q_offset + Tq) : Tk;
  const int64_t lo = window > 0 ? std::max((int64_t)0, q_offset - window + 1) : 0;
  const int64_t tiles = hi > lo ? ceil_div(hi, 64) - lo / 64 : 1;
  const int64_t want = std::max((int64_t)1, ceil_div(512, base));
  return 64 * std::max((int64_t)(dtype == FA_BF16 ? 4 : 2), ceil_div(tiles, want));
}

int64_t n_splits_of(int64_t Tk, int64_t split_keys) { return std::max((int64_t)1, ceil_div(Tk, split_keys)); }

// x: every optional feature, normalised (split_keys 0: no split, > 0: keys per split).
// launch = false: every check, then FA_OK without launching.
fa_status fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                   int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, float scale,
                   int64_t q_offset, int causal, int64_t window, const float *sinks,
                   const float *mask, const fa_strides *strides, fa_dtype dtype, void *stream,
                   const fa_ext &x, bool launch = true) {
  const int64_t split_keys = x.split_keys;
  void *const workspace = x.workspace;
  const size_t workspace_bytes = x.workspace_bytes;
  const bool split = split_keys != 0;
  const bool paged = x.block_table != nullptr;
  // ---- arguments ----
  if (B < 0 || Hq < 0 || Hkv < 0 || Tq < 0 || Tk < 0 || q_offset < 0 || d <= 0) return FA_EINVAL;
  if (!std::isfinite(scale)) return FA_EINVAL;
  if (Hq > 0 && Hkv == 0) return FA_ESHAPE;
  if (Hkv > Hq || (Hkv > 0 && Hq % Hkv != 0)) return FA_ESHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_EUNSUPPORTED;
  if (d != 64 && d != 128) return FA_EUNSUPPORTED;
  // the kernels keep B and Hq in 32 bits; B * Hq * Tq must not overflow
  int64_t rows_total = 0;
  if (B > INT32_MAX || Hq > INT32_MAX || __builtin_mul_overflow(B * Hq, Tq, &rows_total)) return FA_EUNSUPPORTED;
  if (rows_total > 0 && (q == nullptr || o == nullptr)) return FA_EINVAL;
  if (rows_total > 0 && Tk > 0 && (k == nullptr || v == nullptr)) return FA_EINVAL;
  // int32 limits of the kernel's row/key indices and of the 1-D grid
  if (Tq > INT32_MAX - 256 || Tk > INT32_MAX - 256 || q_offset > INT64_MAX / 4 ||
      (window > 0 && window > INT64_MAX / 4))
    return FA_EUNSUPPORTED;

  if (paged) {
    if (x.block_size <= 0 || x.block_size % 64 != 0 || x.block_size > INT32_MAX / 2 || x.num_blocks < 0 ||
        x.num_blocks > INT32_MAX || x.block_table_stride < 0 ||
        x.block_table_stride < (Tk + x.block_size - 1) / x.block_size)
      return FA_EINVAL;
    if (!aligned(x.block_table, 4)) return FA_EUNSUPPORTED;
  }
  if (!(x.softcap >= 0.f) || std::isinf(x.softcap)) return FA_EINVAL;  // NaN, negative or infinite cap
  if (!aligned(x.alibi_slopes, 4)) return FA_EUNSUPPORTED;
  const bool per_seq = x.seqlens_k || x.cu_seqlens_q || x.cu_seqlens_k;
  if (per_seq && q_offset != 0) return FA_EINVAL;  // positions come from the per-sequence lengths
  if (x.cu_seqlens_k && (x.seqlens_k || paged)) return FA_EINVAL;  // one source of key counts
  if ((x.cu_seqlens_q || x.cu_seqlens_k) && strides == nullptr) return FA_EINVAL;  // packed layouts
  if (!aligned(x.seqlens_k, 4) || !aligned(x.cu_seqlens_q, 4) || !aligned(x.cu_seqlens_k, 4))
    return FA_EUNSUPPORTED;

  fa_strides s;
  if (strides) {
    s = *strides;
  } else {
    s.q[0] = Hq * Tq * d; s.q[1] = Tq * d; s.q[2] = d;
    if (paged) {  // pools [num_blocks, Hkv, block_size, d]
      s.k[0] = Hkv * x.block_size * d; s.k[1] = x.block_size * d; s.k[2] = d;
    } else {
      s.k[0] = Hkv * Tk * d; s.k[1] = Tk * d; s.k[2] = d;
    }
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
  if (x.rows_per_block != 0 || x.heads_per_block != 0) {
    rows_pb = x.rows_per_block;
    heads_pb = x.heads_per_block;
    const int64_t waves32 = (int64_t)rows_pb * heads_pb;
    if (rows_pb <= 0 || heads_pb <= 0 || rows_pb % 32 != 0 || group % heads_pb != 0 ||
        (waves32 != 32 && waves32 != 64 && waves32 != 128 && waves32 != 256))
      return FA_EINVAL;
  }
  int64_t n_splits = 0;
  int64_t split_eff = 0;  // keys per split as the kernels take it
  if (split) {
    if (split_keys < 0 || split_keys % 64 != 0) return FA_EINVAL;
    // A split that holds every key is one split whatever its nominal size: cap it there, so the
    // kernels' split arithmetic stays far inside 32 bits for any split_keys.
    split_eff = std::min(split_keys, ceil_div(std::max(Tk, (int64_t)1), 64) * 64);
    n_splits = n_splits_of(Tk, split_eff);
    if (rows_total > 0) {
      if (workspace == nullptr) return FA_EINVAL;
      if (n_splits > INT32_MAX / 4 || rows_total > INT64_MAX / (4 * (d + 2)) / n_splits) return FA_EUNSUPPORTED;
      if ((uint64_t)workspace_bytes < (uint64_t)(n_splits * rows_total * (d + 2) * 4)) return FA_EINVAL;
      if (!aligned(workspace, 16)) return FA_EUNSUPPORTED;
    }
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

  // the tile copies address one (b, KV head) slice of K and of V (paged: one tile) with 32-bit
  // offsets
  if (Tk > 0 && (64 * s.k[2] * es >= INT32_MAX || 64 * s.v[2] * es >= INT32_MAX))
    return FA_EUNSUPPORTED;
  if (Tk > 0 && !paged &&
      (((Tk - 1) * s.k[2] + d) * es >= INT32_MAX || ((Tk - 1) * s.v[2] + d) * es >= INT32_MAX))
    return FA_EUNSUPPORTED;
  const bool auto_geom = rows_pb == 0 && !split;
  if (rows_pb == 0) {
    if (split) split_tiling(group, Tq, &rows_pb, &heads_pb);
    else {
      // a mask shared by every head: 8 waves only where they make 64-row workgroups of 4 heads,
      // whose mask block is staged in LDS
      const bool mask_eight = mask != nullptr && s.mask[1] == 0 && s.mask[3] == 1 && group % 4 == 0 &&
                              group % 8 != 0;
      auto_tiling(B, Hkv, group, Tq,
                  dtype == FA_BF16 && d == 128 && (mask == nullptr || mask_eight) && !(x.softcap > 0.f) &&
                      !x.alibi_slopes && scale > 0.f,
                  &rows_pb, &heads_pb);
      if (dtype == FA_F32 && mask == nullptr && !(x.softcap > 0.f) && !x.alibi_slopes && scale > 0.f &&
          prefer_split_role(B, Hkv, group, Tq, Tk, rows_pb, heads_pb, q_offset, causal, window, cu_count())) {
        rows_pb = 32;  // one-wave blocks: the split-role kernel below
        heads_pb = 1;
      }
    }
  }
  const int nw = (int)((int64_t)rows_pb * heads_pb / 32);
  const int64_t n_row_tiles = (Tq + rows_pb - 1) / rows_pb;
  const int64_t n_blocks = B * Hkv * (group / heads_pb) * n_row_tiles * (split ? n_splits : 1);
  // the merge grid is (ceil(Tq / 4), Hq, B)
  if (n_blocks > INT32_MAX || (split && (Hq > 65535 || B > 65535))) return FA_EUNSUPPORTED;

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
  p.B = (int32_t)B;
  p.Tq = (int32_t)Tq; p.Tk = (int32_t)Tk; p.Hq = (int32_t)Hq; p.Hkv = (int32_t)Hkv;
  p.group = (int32_t)group;
  p.heads_per_block = heads_pb;
  p.rows_per_block = rows_pb;
  p.n_head_groups = (int32_t)(group / heads_pb);
  p.n_row_tiles = (int32_t)n_row_tiles;
  p.n_blocks = (int32_t)n_blocks;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * kLog2e;
  p.inv_scale = 1.f / scale;
  p.mask_vec = mask != nullptr && s.mask[3] == 1 && aligned(mask, 16) && s.mask[0] % 4 == 0 &&
               s.mask[1] % 4 == 0 && s.mask[2] % 4 == 0;
  p.tile_major = 0;
  if (mask != nullptr && s.mask[0] == 0 && s.mask[1] == 0) {
    // slices (without head groups) per block: the largest divisor of their count up to
    // FA_MASK_SLICE_BLOCK, which balances mask re-reads against K/V re-reads
    const int64_t n_sl = B * Hkv * (split ? n_splits : 1);
    int sb = 1;
    for (int c = FA_MASK_SLICE_BLOCK; c >= 1; --c)
      if (n_sl % c == 0) { sb = c; break; }
    p.tile_major = sb;
  }
  p.n_splits = (int32_t)n_splits;
  p.split_tiles = split ? (int32_t)(split_eff / 64) : 0;
  p.ws_acc = split ? static_cast<float *>(workspace) : nullptr;
  p.ws_ml = split ? static_cast<float *>(workspace) + n_splits * rows_total * d : nullptr;
  p.block_table = x.block_table;
  p.bt_stride = paged ? x.block_table_stride : 0;
  p.block_size = paged ? (int32_t)x.block_size : 0;
  p.num_blocks = paged ? (int32_t)x.num_blocks : 0;
  p.seqlens_k = x.seqlens_k;
  p.cu_seqlens_q = x.cu_seqlens_q;
  p.cu_seqlens_k = x.cu_seqlens_k;
  p.Tq_all = (int32_t)Tq;
  p.cap_in = x.softcap > 0.f ? scale / x.softcap : 0.f;
  p.cap_out = x.softcap > 0.f ? x.softcap * kLog2e : 0.f;
  p.alibi = x.alibi_slopes;
  p.q_start = 0;
  p.k_start = 0;

  const bool bf16 = dtype == FA_BF16;
  // MODE 2-4 for the score variants: 2 with a mask, else 3 (softcap, with or without ALiBi) or
  // 4 (ALiBi alone).  MODE 2 also serves a scale that is not positive (the raw-maximum form
  // of MODE 0 and 1 needs scale > 0).  MODE 1 for an additive mask, MODE 0 without.
  const int mode = (x.softcap > 0.f || x.alibi_slopes) ? (mask != nullptr ? 2 : x.softcap > 0.f ? 3 : 4)
                   : !(scale > 0.f) ? 2 : mask != nullptr ? 1 : 0;
  // stage the mask through LDS when the workgroup's rows share mask rows across its heads and
  // their count is the one the kernel stages (64 for 8 waves, else 32)
  const int64_t mask_rows = nw == 8 ? 64 : 32;
  p.mask_lds = mode == 1 && mask != nullptr && p.mask_vec && s.mask[1] == 0 && rows_pb == mask_rows &&
               mask_rows * s.mask[2] * 4 < INT32_MAX;
  KernelFn fn = bf16 ? (d == 64 ? pick_nw<true, 64>(nw, mode) : pick_nw<true, 128>(nw, mode))
                     : (d == 64 ? pick_nw<false, 64>(nw, mode) : pick_nw<false, 128>(nw, mode));
  // A plain fp32 call that one-wave workgroups already spread over the CUs is bound by each
  // block's serial chain of fp32 MFMAs: there the split-role kernel runs each 32-row block on
  // 4 waves (two computing scores a tile ahead, two the softmax and PV for half of d each; the
  // same bits).
  int waves = nw;
  if (auto_geom && !bf16 && mode == 0 && nw == 1) {
    waves = 5;
    fn = d == 64 ? fa_fwd_so_kernel<64> : fa_fwd_so_kernel<128>;
  }
  // The plain 8-wave bf16 kernel over several rounds of workgroups runs persistent: one
  // workgroup per CU walks its share of the work items (the same bits; ≈ 1 % faster on the
  // 8,192-token causal batch than one workgroup per item).
  unsigned grid = (unsigned)n_blocks;
  if (fn == pick_nw<true, 128>(8, 0) && !split && !paged && !p.seqlens_k && !p.cu_seqlens_q && !p.cu_seqlens_k &&
      Tk % 64 == 0) {
    const int ncu = cu_count();
    if (ncu >= 8 && ncu % 8 == 0 && n_blocks >= 2 * (int64_t)ncu) {
      fn = fa_fwd_kernel<true, 128, 8, 0, 1, true>;
      grid = (unsigned)ncu;
    }
  }
  if (!launch) return FA_OK;
  (void)hipGetLastError();  // clear a stale error so the check below reports this launch
  hipLaunchKernelGGL(fn, dim3(grid), dim3(waves * 64), 0, static_cast<hipStream_t>(stream), p);
  if (hipGetLastError() != hipSuccess) return FA_EDEVICE;
  if (split) {  // merge the splits' row states into o and lse (same stream, so after the above)
    void (*merge)(Params) = bf16 ? (d == 64 ? fa_merge_kernel<true, 64> : fa_merge_kernel<true, 128>)
                                 : (d == 64 ? fa_merge_kernel<false, 64> : fa_merge_kernel<false, 128>);
    hipLaunchKernelGGL(merge, dim3((unsigned)((Tq + 3) / 4), (unsigned)Hq, (unsigned)B), dim3(256), 0,
                       static_cast<hipStream_t>(stream), p);
    if (hipGetLastError() != hipSuccess) return FA_EDEVICE;
  }
  return FA_OK;
}

// ---------------------------------------------------------------------------------------
// Scratch for fa_fwd_splitkv_noalloc: the split-KV workspace of callers that cannot allocate
// device memory.  Every GPU the library runs on holds its own copy of this array until the
// process ends.  In host code its name is only a stand-in: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and is the only form
// handed to kernels.
// ---------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(FA_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device.
fa_status scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return FA_EDEVICE;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                 int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, float scale,
                 int64_t q_offset, int causal, int64_t window, const float *sinks,
                 const float *mask, const fa_strides *strides, fa_dtype dtype, void *stream) {
  const fa_ext x = {};
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks,
                  mask, strides, dtype, stream, x);
}

fa_status fa_fwd_ext(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                     int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, float scale,
                     int64_t q_offset, int causal, int64_t window, const float *sinks,
                     const float *mask, const fa_strides *strides, fa_dtype dtype, void *stream,
                     const fa_ext *ext) {
  fa_ext x = {};
  if (ext) {
    if (ext->size < sizeof(uint32_t)) return FA_EINVAL;
    std::memcpy(&x, ext, std::min((size_t)ext->size, sizeof(fa_ext)));
  }
  if (x.split_keys < -1) return FA_EINVAL;
  if (x.split_keys == -1)
    x.split_keys = default_split_keys(
        B, Hq, Hkv, Tq, Tk,
        (x.seqlens_k || x.cu_seqlens_q || x.cu_seqlens_k) ? std::max((int64_t)0, Tk - Tq) : q_offset, causal,
        window, dtype);
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks,
                  mask, strides, dtype, stream, x);
}

fa_status fa_fwd_tiled(const void *q, const void *k, const void *v, void *o, float *lse,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                       float scale, int64_t q_offset, int causal, int64_t window,
                       const float *sinks, const float *mask, const fa_strides *strides,
                       fa_dtype dtype, void *stream, const fa_tiling *tiling) {
  fa_ext x = {};
  if (tiling) { x.rows_per_block = tiling->rows_per_block; x.heads_per_block = tiling->heads_per_block; }
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks,
                  mask, strides, dtype, stream, x);
}

fa_status fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                          float scale, int64_t q_offset, int causal, int64_t window,
                          const float *sinks, const float *mask, const fa_strides *strides,
                          fa_dtype dtype, void *stream, const fa_tiling *tiling, int64_t split_keys,
                          void *workspace, size_t workspace_bytes) {
  if (split_keys == 0) split_keys = default_split_keys(B, Hq, Hkv, Tq, Tk, q_offset, causal, window, dtype);
  if (split_keys <= 0) return FA_EINVAL;
  fa_ext x = {};
  if (tiling) { x.rows_per_block = tiling->rows_per_block; x.heads_per_block = tiling->heads_per_block; }
  x.split_keys = split_keys;
  x.workspace = workspace;
  x.workspace_bytes = workspace_bytes;
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks,
                  mask, strides, dtype, stream, x);
}

fa_status fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                                  float scale, int64_t q_offset, int causal, int64_t window,
                                  const float *sinks, const float *mask, const fa_strides *strides,
                                  fa_dtype dtype, void *stream, const fa_tiling *tiling, int64_t split_keys) {
  if (split_keys == 0) split_keys = default_split_keys(B, Hq, Hkv, Tq, Tk, q_offset, causal, window, dtype);
  if (split_keys <= 0) return FA_EINVAL;
  // the workspace this call needs (0 for arguments the checks below reject); its contents on
  // entry do not matter, so nothing has to be cleared
  const size_t need = fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, split_keys);
  if (need > kScratchBytes) return FA_ESCRATCH;
  fa_ext x = {};
  if (tiling) { x.rows_per_block = tiling->rows_per_block; x.heads_per_block = tiling->heads_per_block; }
  x.split_keys = split_keys;
  x.workspace_bytes = kScratchBytes;
  // every argument check first (against a stand-in workspace address that nothing reads), so
  // that errors do not depend on the device
  x.workspace = reinterpret_cast<void *>(uintptr_t(256));
  fa_status st = fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks,
                          mask, strides, dtype, stream, x, false);
  if (st != FA_OK) return st;
  if (fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, split_keys) == 0) {  // no rows: nothing to launch
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks, mask,
                    strides, dtype, stream, x);
  }
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != FA_OK) return st;
  x.workspace = ws;
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks,
                  mask, strides, dtype, stream, x);
}

int64_t fa_splitkv_default_keys(int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk,
                                int64_t q_offset, int causal, int64_t window, fa_dtype dtype) {
  return default_split_keys(B, Hq, Hkv, Tq, Tk, q_offset, causal, window, dtype);
}

size_t fa_splitkv_workspace_bytes(int64_t B, int64_t Hq, int64_t Tq, int64_t Tk, int64_t d,
                                  int64_t split_keys) {
  if (B < 0 || Hq < 0 || Tq < 0 || Tk < 0 || d <= 0 || split_keys <= 0) return 0;
  int64_t rows = 0;
  if (__builtin_mul_overflow(B, Hq, &rows) || __builtin_mul_overflow(rows, Tq, &rows)) return 0;
  const int64_t ns = n_splits_of(Tk, split_keys);
  if (rows > 0 && (ns > INT64_MAX / (4 * (d + 2)) / rows)) return 0;
  return (size_t)(ns * rows * (d + 2) * 4);
}

const char *fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_EINVAL: return "invalid argument";
    case FA_ESHAPE: return "invalid head shape (Hq must be a positive multiple of Hkv)";
    case FA_EUNSUPPORTED: return "unsupported (d must be 64 or 128; dtype fp32 or bf16; aligned tensors)";
    case FA_EDEVICE: return "device launch failed";
    case FA_ESCRATCH: return "the call needs more workspace than the no-allocation scratch holds";
  }
  return "unknown status";
}

}  // extern "C"
