/*
 * fa.h -- C ABI of libfa.so, the tiled FlashAttention forward pass for AMD MI355X (gfx950).
 *
 * The operation ("FlashAttention forward in C", tinyllm L9.3, section 2.1 "What is
 * computed", with the additive mask of "Fused attention and softmax: fast and exact",
 * OneModel, "What is computed"): for every sequence b, query head h and query row i,
 *
 *   p_i  = q_offset + i                                   (absolute position of row i)
 *   V_i  = { j < Tk : (causal == 0 or j <= p_i) and (window <= 0 or j > p_i - window) }
 *   s_ij = scale * q_i . k_j + mask[b, h, i, j]           (mask term 0 without a mask)
 *   o_i  = sum_{j in V_i} e^{s_ij} v_j / (sum_{j in V_i} e^{s_ij} + e^{z_h})
 *   lse_i = log(sum_{j in V_i} e^{s_ij} + e^{z_h})        (natural log)
 *
 * where head h reads KV head floor(h / (Hq / Hkv)) (grouped-query attention) and the
 * e^{z_h} sink term is present only when `sinks` is given.  A mask entry of -inf removes
 * the key.  A row with no visible key and no sink gets o = 0 and lse = -inf.  With a mask and
 * scale > 0 the score is formed as scale * (q_i . k_j + mask / scale), the mask term being
 * the starting value of the dot product's accumulator: the same value up to fp32 rounding,
 * except that a finite entry above FLT_MAX * scale overflows to +inf there (as a +inf entry,
 * it makes its row NaN).

 *
 * It is computed one absolute key tile [64t, 64t + 64) at a time with the online softmax
 * of "FlashAttention forward in C" section 2.2 (and "IV.5: Flash attention", "Softmax
 * without seeing the whole row"); the score matrix is never stored.  Key tiles sit at
 * absolute positions and each row skips tiles it cannot see (section 2.4), so the bits of
 * row i depend only on q_i, K, V, p_i, the flags, d and the dtype: not on how the queries
 * are chunked (q_offset), on the query tile, the batch, the strides or the launch order.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_EINVAL = 1,       /* bad argument: negative size or q_offset, NULL tensor, bad stride, non-finite scale */
  FA_ESHAPE = 2,       /* head shapes: Hkv == 0 with Hq > 0, Hkv > Hq, or Hq % Hkv != 0 */
  FA_EUNSUPPORTED = 3, /* d not 64 or 128, unknown dtype, misaligned tensor, size beyond int32 */
  FA_EDEVICE = 4,      /* the HIP launch failed (no device, invalid stream, ...) */
  FA_ESCRATCH = 5      /* fa_fwd_splitkv_noalloc: the call needs more than FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

typedef enum {
  FA_F32 = 0,  /* q, k, v, o are fp32; all arithmetic fp32 */
  FA_BF16 = 1  /* q, k, v, o are bf16; scores and accumulators fp32, weights rounded to bf16 */
} fa_dtype;

/*
 * Element strides.  The d axis of q, k, v and o is contiguous (stride 1); the t axis of
 * lse is contiguous.  Strides must be >= 0.  A stride of 0 in mask broadcasts that axis.
 */
typedef struct {
  int64_t q[3], k[3], v[3], o[3]; /* along (b, h, t) */
  int64_t lse[2];                 /* along (b, h) */
  int64_t mask[4];                /* along (b, h, i, j); i is the row of this call */
} fa_strides;

/*
 * fa_fwd -- enqueue the forward pass on `stream` and return; results are valid once the
 * stream has synchronised.
 *
 * Pointers are device memory owned by the caller:
 *   q     [B, Hq,  Tq, d]  dtype       k, v [B, Hkv, Tk, d]  dtype
 *   o     [B, Hq,  Tq, d]  dtype (written)
 *   lse   [B, Hq,  Tq]     fp32 (written) or NULL
 *   sinks [Hq]             fp32 raw logits (not scaled) or NULL
 *   mask  fp32 additive mask indexed [b, h, i, j] through strides->mask, or NULL
 * strides == NULL means contiguous [B, H, T, d] tensors, lse [B, Hq, Tq] and a mask of
 * [Tq, Tk] broadcast over b and h.  scale is taken as given (callers usually pass
 * 1/sqrt(d) rounded to fp32).  window <= 0 means no window.  stream is a hipStream_t
 * (NULL: the default stream).
 *
 * Alignment: q, k, v and their (b, h, t) strides must be 16-byte aligned; o and its
 * strides 16-byte aligned for fp32, 8-byte for bf16.
 *
 * The library allocates nothing and keeps no state: scratch is on-chip (LDS and
 * registers) and its size does not depend on Tk.  Calls on different streams may overlap.
 *
 * A row with no visible key and no sink gets o = +0 (sign bit clear) and lse = -inf; every
 * zero in o is written as +0.
 *
 * Errors are returned synchronously, before any launch, and leave o and lse untouched:
 * FA_EINVAL, FA_ESHAPE and FA_EUNSUPPORTED as listed in fa_status.  B * Hq * Tq == 0 returns
 * FA_OK without a launch.  Tk == 0 is valid (k and v may then be NULL): every row gets
 * o = 0 and lse = -inf, or lse = the sink logit.  FA_EDEVICE reports a failed launch.
 */
fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                 float scale, int64_t q_offset, int causal, int64_t window,
                 const float *sinks, const float *mask, const fa_strides *strides,
                 fa_dtype dtype, void *stream);

/*
 * Launch geometry.  A workgroup covers `rows_per_block` consecutive query rows of
 * `heads_per_block` query heads that share one KV head, so each K/V tile staged on chip
 * serves all of them.  rows_per_block * heads_per_block must be 32, 64, 128 or 256 (one wave
 * per 32 rows of one head); heads_per_block must divide Hq / Hkv.  0 in both fields picks
 * automatically (what fa_fwd does).
 */
typedef struct {
  int32_t rows_per_block;
  int32_t heads_per_block;
} fa_tiling;

/*
 * fa_fwd_tiled -- fa_fwd with an explicit launch geometry (tiling may be NULL).  The
 * results are bit-identical to fa_fwd's for every valid geometry: the geometry only
 * decides which rows share a workgroup ("FlashAttention forward in C", section 2.4:
 * results do not depend on the query tile size).  An invalid geometry returns FA_EINVAL.
 */
fa_status fa_fwd_tiled(const void *q, const void *k, const void *v, void *o, float *lse,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                       float scale, int64_t q_offset, int causal, int64_t window,
                       const float *sinks, const float *mask, const fa_strides *strides,
                       fa_dtype dtype, void *stream, const fa_tiling *tiling);

/*
 * Split-KV ("FlashAttention forward in C", "Going further": split-KV / Flash-Decoding).  For
 * calls with few query rows and many keys (decoding: Tq = 1, q_offset = Tk - 1), where one
 * workgroup per query tile leaves most of the GPU idle, the keys are cut into splits of
 * `split_keys` keys at absolute positions [s * split_keys, (s + 1) * split_keys).  One kernel
 * runs every (query tile, split) pair and keeps each row's online-softmax state (m, l, a) of
 * its split; a second kernel merges the splits of each row with the tile rescale, in
 * ascending split order:
 *
 *   M = max_s m_s,  l = sum_s e^{m_s - M} l_s,  a = sum_s e^{m_s - M} a_s,  o = a / l,
 *   lse = M + ln l                      (splits with l_s = 0 are left out; the sink term
 *                                        belongs to split 0)
 *
 * which is the same o and lse as fa_fwd up to rounding (the pages: trading invariance for
 * parallelism).  The bits of a row depend on q_i, K, V, p_i, the flags, d, the dtype and
 * split_keys only: not on chunking, tiling, batch, strides or launch order.  With a single
 * split (split_keys >= Tk) the results equal fa_fwd's bit for bit.  (Every entry point writes
 * a zero output as +0.)
 *
 * Arguments as for fa_fwd_tiled, plus:
 *   split_keys       keys per split, a positive multiple of 64; 0 picks
 *                    fa_splitkv_default_keys(...).  Anything else returns FA_EINVAL.  Any
 *                    value >= Tk (up to INT64_MAX) is one split.
 *   workspace        device memory owned by the caller, 16-byte aligned, at least
 *                    fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, split_keys) bytes (else
 *                    FA_EINVAL; misaligned: FA_EUNSUPPORTED).  Its contents on entry do not
 *                    matter; it holds the per-split row states afterwards.  Calls that
 *                    overlap in time need workspaces of their own.
 * Both kernels are enqueued on `stream`; the library allocates nothing.  B and Hq must be at
 * most 65,535 (else FA_EUNSUPPORTED).  A row whose visible keys lie in one split (and, with
 * a sink, in split 0) is finished by that split's kernel; only the others go through the merge.
 */
fa_status fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                         float scale, int64_t q_offset, int causal, int64_t window,
                         const float *sinks, const float *mask, const fa_strides *strides,
                         fa_dtype dtype, void *stream, const fa_tiling *tiling, int64_t split_keys,
                         void *workspace, size_t workspace_bytes);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call without the workspace arguments.  The workspace is a static device array inside
 * the library, FA_NOALLOC_SCRATCH_BYTES bytes on each GPU it runs on, held until the process
 * ends; the call allocates nothing and calls no allocating routine.  Results equal
 * fa_fwd_splitkv's with the same split_keys bit for bit.
 *
 * Arguments as for fa_fwd_splitkv (split_keys 0: the default split).  A call whose workspace,
 * fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, split_keys), exceeds FA_NOALLOC_SCRATCH_BYTES
 * returns FA_ESCRATCH before any launch; other errors as for fa_fwd_splitkv.  The array is
 * shared by every call on a GPU and keeps the last call's contents (no call depends on them):
 * calls that overlap in time on one GPU, on any streams, race on it and must not be issued.
 * The stream must belong to the current device, whose array the call uses.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
fa_status fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                                 float scale, int64_t q_offset, int causal, int64_t window,
                                 const float *sinks, const float *mask, const fa_strides *strides,
                                 fa_dtype dtype, void *stream, const fa_tiling *tiling, int64_t split_keys);

/*
 * The split size fa_fwd_splitkv takes for split_keys = 0: a multiple of 64 (at least 256 for
 * bf16, 128 for fp32) that cuts the keys some row can see into enough splits to give a
 * 256-CU device about 512 workgroups.  It depends on the arguments only, not on the device.
 */
int64_t fa_splitkv_default_keys(int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk,
                                int64_t q_offset, int causal, int64_t window, fa_dtype dtype);

/*
 * Workspace bytes fa_fwd_splitkv needs: (d + 2) * 4 bytes per (split, row), with
 * max(1, ceil(Tk / split_keys)) splits and B * Hq * Tq rows.  0 for invalid arguments.
 */
size_t fa_splitkv_workspace_bytes(int64_t B, int64_t Hq, int64_t Tq, int64_t Tk, int64_t d,
                                  int64_t split_keys);

/*
 * Optional features of fa_fwd_ext, combinable with each other and with every flag of fa_fwd.
 * Zero-initialise the struct and set `size` to sizeof(fa_ext); a field left at zero is off.
 *
 * Geometry: rows_per_block, heads_per_block as in fa_tiling.
 *
 * Split-KV: split_keys 0 = no split; > 0 = keys per split (a multiple of 64); -1 = the
 *   default of fa_splitkv_default_keys (for per-sequence key counts, with q_offset = Tk - Tq).
 *   workspace and workspace_bytes as for fa_fwd_splitkv.
 *
 * Paged K/V ("FlashAttention forward in C", "Key Takeaways": paged attention for decode
 *   performs the same tile update on blocks, held bit for bit to this kernel).  When
 *   block_table is not NULL, k and v are pools of num_blocks blocks of block_size keys (a
 *   positive multiple of 64), indexed [block, KV head, key in block, d] through strides->k
 *   and strides->v, whose first entry then steps from block to block (strides == NULL:
 *   contiguous [num_blocks, Hkv, block_size, d] pools).  Key j of sequence b is row
 *   j % block_size of block block_table[b * block_table_stride + j / block_size].
 *   block_table (device int32) needs valid entries for the blocks holding keys [0, Tk) of
 *   each sequence (or [0, seqlens_k[b])); block_table_stride >= ceil(Tk / block_size).  A
 *   block index outside [0, num_blocks) reads as zero keys and values (never out of
 *   bounds).  The results equal fa_fwd's on the same keys laid out contiguously, bit for bit.
 *
 * Per-sequence key counts: seqlens_k (device int32 [B]) or NULL.  Sequence b then has
 *   n_b = min(max(seqlens_k[b], 0), Tk) keys and its Tq query rows are its last Tq positions:
 *   row i sits at p_i = n_b - Tq + i (rows with p_i < 0 see no key when causal).  q_offset
 *   must be 0.  Row i of sequence b then equals fa_fwd with Tk = n_b and q_offset = n_b - Tq
 *   (when that is >= 0), bit for bit.
 *
 * Packed sequences (varlen batching: candle's B > 1 path; the batch invariance of
 *   "FlashAttention forward in C" section 4): cu_seqlens_q and/or cu_seqlens_k (device int32
 *   [B + 1], non-decreasing prefix sums starting at 0) or NULL.  Sequence b's query rows are
 *   tokens [cu_seqlens_q[b], cu_seqlens_q[b + 1]) of q, o and lse (m_b of them, at most Tq),
 *   its keys tokens [cu_seqlens_k[b], cu_seqlens_k[b + 1]) of k and v (n_b, at most Tk); the
 *   tensors are indexed by token through the t strides and the b strides are not used (q, o:
 *   [total_q, Hq, d] is strides {0, d, Hq d}; lse [Hq, total_q] is {0, total_q}), so strides
 *   must be given.  Row i of sequence b sits at p_i = n_b - m_b + i (p_i = i when m_b = n_b)
 *   and q_offset must be 0.  cu_seqlens_k excludes seqlens_k and paging (which take their key
 *   counts from seqlens_k).  Every row equals a single-sequence fa_fwd call on its own
 *   tokens with q_offset = n_b - m_b, bit for bit.  The offsets live in device memory, so
 *   the library cannot check them: lengths are clamped to [0, Tq] and [0, Tk], but offsets
 *   that put a sequence's tokens outside q, k, v, o or lse make the kernels read or write out
 *   of bounds (the caller's error, as for any pointer argument).
 *
 * Score variants (the candle page, "KV 缓存与注意力", attention/: variants with ALiBi and
 *   softcap; their usual definitions): softcap c > 0 turns the logit x = scale * q.k into
 *   c * tanh(x / c) (0: off; negative, NaN or infinite: FA_EINVAL); alibi_slopes (device fp32
 *   [Hq] or NULL) adds -slope_h * |p_i - j| to the score, p_i the row's absolute position (the
 *   distance counts keys on either side).  The score becomes
 *     s_ij = [c tanh(scale q_i.k_j / c)] - slope_h |p_i - j| + mask[b, h, i, j].
 *   Both keep every property above (chunking, tiling, batch, paging, split-KV).
 */
typedef struct {
  uint32_t size;                  /* sizeof(fa_ext) */
  int32_t rows_per_block;         /* launch geometry (0, 0: automatic) */
  int32_t heads_per_block;
  int32_t reserved;               /* 0 */
  int64_t split_keys;             /* 0: no split; > 0: keys per split; -1: default */
  void *workspace;                /* split-KV workspace (device) */
  size_t workspace_bytes;
  const int32_t *block_table;     /* paged K/V (device) or NULL */
  int64_t block_table_stride;     /* entries between consecutive sequences' rows */
  int64_t block_size;             /* keys per block */
  int64_t num_blocks;             /* blocks in each pool */
  const int32_t *seqlens_k;       /* per-sequence key counts (device) or NULL */
  const int32_t *cu_seqlens_q;    /* packed query rows: prefix sums [B + 1] (device) or NULL */
  const int32_t *cu_seqlens_k;    /* packed keys: prefix sums [B + 1] (device) or NULL */
  float softcap;                  /* logit cap c > 0, or 0 for none */
  int32_t reserved2;              /* 0 */
  const float *alibi_slopes;      /* [Hq] fp32 ALiBi slopes (device) or NULL */
} fa_ext;

/*
 * fa_fwd_ext -- fa_fwd with the optional features of `ext` (NULL: none).  Arguments as for
 * fa_fwd; Tk is the largest key count (with paging: the logical sequence length the block
 * table spans).  Errors as for fa_fwd, plus FA_EINVAL for an inconsistent ext (size too small,
 * split_keys < -1 or not a multiple of 64, block_size not a positive multiple of 64,
 * block_table_stride too short, q_offset != 0 with per-sequence lengths, cu_seqlens_k with
 * seqlens_k or paging, packed sequences without strides, a missing or short workspace)
 * and FA_EUNSUPPORTED for a misaligned block table, length array or workspace.
 */
fa_status fa_fwd_ext(const void *q, const void *k, const void *v, void *o, float *lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                     float scale, int64_t q_offset, int causal, int64_t window,
                     const float *sinks, const float *mask, const fa_strides *strides,
                     fa_dtype dtype, void *stream, const fa_ext *ext);

/* Static English name of a status code (never NULL). */
const char *fa_status_str(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
