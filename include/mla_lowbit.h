/*
 * mla_lowbit.h -- C ABI of libmla_lowbit.so: native low-bit MLA decode
 * (QuantMLA-style C4R4 / C2R4 caches) for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [QuantMLA x]  "QuantMLA: Function-Aligned Dual-Path Quantization for
 *                 Low-Bit MLA KV Caching", section x.
 *   [MLA blog x]  "DeepSeek MLA: low-rank KV cache and inference efficiency"
 *                 (weigao.cc), section x.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *     memory, including workspaces; the library allocates nothing and keeps
 *     no state between calls.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Results are visible after the caller synchronizes.
 *   - Return value: MLA_LB_OK (0) or a negative error code.  Shape, pointer
 *     and size checks run on the host BEFORE any HIP call, so a rejected call
 *     touches neither the GPU nor its arguments.  A failed launch returns
 *     MLA_LB_EHIP.  No exception crosses the ABI.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Device-side guards: tokens whose slot / sequence slot / page id fall
 *     outside the sizes passed in are skipped (never dereferenced).  Such
 *     inputs give unspecified results, not memory faults.  NaN/Inf inputs and
 *     overlapping slots are outside the defined domain.
 *   - Numeric domain of the decode calls: the softmax keeps one reference
 *     maximum per head and split, fixed by its first tile, and lets later
 *     weights exp(S - reference) grow up to 2^64 before the reference is
 *     raised (the split is then redone; the result is the same single
 *     softmax).  The fp32 sums of weighted latent values therefore need
 *     |c~_i| * seq_len < 2^63 (about 9.2e18) to stay finite -- 2^64 less
 *     headroom than a softmax rescaled at every tile.  Within that domain
 *     every finite input gives finite outputs.
 *
 * Cache format (one physical page = 64 token slots; slot = page*64 + offset)
 *   [QuantMLA App. C.4/C.5], [MLA blog §6].  Structure-of-arrays, every
 *   region starting at a multiple of 256 bytes:
 *     codes_c  C4R4: [4 blk][64 tok][64 B], blk = content dims 128*blk..+127,
 *                    byte k holds dims 2k (bits 0-3) and 2k+1 (bits 4-7)
 *              C2R4: [2 blk][64 tok][64 B], blk = content dims 256*blk..+255,
 *                    little-endian 32-bit word k holds dims 16k..16k+15:
 *                    dim 16k+2m in bits 2m..2m+1, dim 16k+2m+1 in bits
 *                    16+2m..17+2m (m = 0..7)
 *     codes_r  [64 tok][32 B], byte k holds RoPE dims 2k (lo) and 2k+1 (hi)
 *     meta_c   [64 tok][8 groups][scale, zero] bf16
 *     meta_r   [64 tok][scale, zero] bf16; C4R4F: [64 tok][scale, zero]
 *              fp32 (content regions as C4R4)
 *   Page bytes: C4R4 20736 (324 per token), C2R4 12544 (196 per token),
 *   C4R4F 20992 (328 per token).
 *
 * Quantizer [QuantMLA §4.1, App. C.4] (per token, per group of 64 values x,
 * m = 2^bits - 1, all arithmetic IEEE fp32, round-to-nearest-even):
 *     s = bf16(fl32(fl32(max x - min x) / m)),  z = min x (bf16-exact),
 *     q = clamp(rint(fl32(fl32(x - z) / s)), 0, m), or q = 0 when s == 0,
 *     reconstruction x^ = bf16(fl32(q * s + z)).
 * Content groups use bits 4 (C4R4, C4R4F) or 2 (C2R4); the RoPE group uses
 * 4 bits.  C4R4F's RoPE group keeps fp32 metadata instead:
 *     s = fl32(fl32(max x - min x) / 15),  z = min x,
 *     q = clamp(rint(fl32(fl32(x - z) / s)), 0, 15), or q = 0 when s == 0,
 *     reconstruction x^ = bf16(fl32(fl32(q * s) + z))  (product rounded first).
 *
 * BF16 protection buffer [QuantMLA §3.3, App. C.5]: per sequence slot,
 * prot[132][576] bf16, a row = [c (512) | k_R (64)].  Token position i < 4
 * uses row i; i >= 4 uses row 4 + (i mod 128).  For a sequence of length L
 * the protected set is [0, min(4,L)) U [max(0, L-128), L): those tokens are
 * read from prot, all others from their packed copy.
 */
#ifndef MLA_LOWBIT_H
#define MLA_LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache formats, CxRy = x-bit content cache, y-bit RoPE-key cache
 * [QuantMLA §4.1].  MLA_LB_C4R4F is C4R4 with the RoPE group's scale and
 * zero kept in fp32, as the pages store RoPE scales [QuantMLA App. C.4/C.5]. */
typedef enum { MLA_LB_C4R4 = 0, MLA_LB_C2R4 = 1, MLA_LB_C4R4F = 2 } mla_lb_format;

enum {
  MLA_LB_OK = 0,
  MLA_LB_EINVAL = -1,     /* null pointer or invalid scalar argument */
  MLA_LB_ESHAPE = -2,     /* unsupported or inconsistent sizes       */
  MLA_LB_EFORMAT = -3,    /* unknown mla_lb_format                   */
  MLA_LB_EWORKSPACE = -4, /* workspace missing or too small          */
  MLA_LB_EHIP = -5        /* HIP runtime error at launch             */
};

enum {
  MLA_LB_D_C = 512,        /* content latent width  [MLA blog §1]      */
  MLA_LB_D_R = 64,         /* RoPE key width        [MLA blog §3]      */
  MLA_LB_PAGE_TOKENS = 64, /* tokens per page       [QuantMLA App. C.5] */
  MLA_LB_PROT_ROWS = 132,  /* 4 sink + 128 recent   [QuantMLA App. C.5] */
  MLA_LB_MAX_HEADS = 128,
  MLA_LB_MAX_ROWS = 65536, /* queries x heads per sequence (mla_decode_lowbit_mq): a
                              512-token prefill chunk at 128 heads */
  MLA_LB_NOALLOC_SCRATCH_BYTES = 64 << 20  /* per-GPU scratch of mla_decode_lowbit_noalloc */
};

/* Library ABI version (host, pure). */
int mla_lb_version(void);

/* Static message for an error code (host, pure, never NULL). */
const char* mla_lb_strerror(int code);

/* Bytes of one physical page of format f (20736 / 12544 / 20992), 0 if f is unknown
 * (host, pure). */
size_t mla_lb_page_bytes(int f);

/* Bytes of one sequence slot's protection buffer: 132*576*2 = 152064
 * (host, pure). */
size_t mla_lb_prot_bytes_per_seq(void);

/*
 * kv_quant_append -- the fused cache writer [QuantMLA App. C.5]: quantize
 * each new token's content latent and post-RoPE key in groups of 64, pack the
 * codes and the bf16 (scale, zero) metadata into its slot, and refresh the
 * BF16 protection buffer.  A packed copy is written for every token, including
 * protected ones, so a token leaving the recent window switches to its packed
 * copy with no requantization.
 *
 *   latent       [T][512] bf16   content latent c of each token
 *   k_rope       [T][64]  bf16   decoupled RoPE key, already rotated
 *   slot_mapping [T] int64       physical page * 64 + offset; must be in
 *                                [0, num_pages*64); distinct within a call
 *   seq_slot     [T] int32       protection-buffer slot of the token's sequence,
 *                                in [0, num_seq_slots)
 *   pos          [T] int32       zero-based position of the token in its sequence
 *   new_len      [T] int32       length of the token's sequence once every token
 *                                of this call is in.  The bf16 row of token
 *                                `pos` is written iff pos is in the protected set
 *                                of that length, so a call may carry many tokens
 *                                of one sequence (a whole prompt) without two of
 *                                them racing for a ring row.
 *   T            >= 0 tokens (T == 0 is a no-op)
 *   pages        [num_pages][page_bytes(f)] bytes (written at the token slots)
 *   prot         [num_seq_slots][132][576] bf16 (rows written as above)
 * Tokens with an out-of-range slot, seq_slot, or pos < 0 are skipped.
 */
int kv_quant_append(int f, const uint16_t* latent, const uint16_t* k_rope,
                    const int64_t* slot_mapping, const int32_t* seq_slot,
                    const int32_t* pos, const int32_t* new_len, int32_t T,
                    uint8_t* pages, int64_t num_pages, uint16_t* prot,
                    int32_t num_seq_slots, void* stream);

/*
 * mla_decode_lowbit_workspace -- bytes of workspace mla_decode_lowbit needs
 * for the same (f, B, H, max_seq_len, num_splits) (host).  Zero when the
 * call runs in one pass (a single split per sequence).  The automatic plan
 * (num_splits = 0) sizes itself to the compute units of the current HIP
 * device (256 when no device is visible), so query it with the device the
 * decode call will run on current.
 *   bytes (host out)
 */
int mla_decode_lowbit_workspace(int f, int32_t B, int32_t H, int32_t max_seq_len,
                                int32_t num_splits, size_t* bytes);

/*
 * mla_decode_lowbit -- decode attention over the mixed-precision cache
 * [QuantMLA §3.3, App. C.5], absorbed MLA form [MLA blog §4]:
 *
 *   S[b,h,i] = softmax_scale * (q_lat[b,h] . c~_i + q_rope[b,h] . k~_R,i)
 *   out[b,h] = sum_i softmax_i(S[b,h,:]) c~_i          (512-d latent output)
 *   lse[b,h] = ln sum_i exp(S[b,h,i])
 *
 * over i in [0, seq_lens[b]), one global softmax per (b, h), where
 * (c~_i, k~_R,i) is the protected bf16 row for i in the protected set and the
 * reconstruction from the packed copy otherwise.  Packed codes are unpacked
 * and dequantized inside the kernel; no bf16 history or per-head K/V is
 * formed.  Scores and aggregation run on bf16 matrix cores with fp32
 * accumulation.  The sequence is split across compute units and the partial
 * (max, sum, unnormalised output) triples are merged by the log-sum-exp rule
 * [QuantMLA App. C.5, App. F.1 (split-result combination)].
 *
 *   q_lat        [B][H][512] bf16   absorbed query (W_UK^T q^C)
 *   q_rope       [B][H][64]  bf16   post-RoPE query part
 *   pages, num_pages, prot, num_seq_slots: as in kv_quant_append
 *   seq_slot     [B] int32          protection-buffer slot of each sequence
 *   block_table  [B][max_blocks] int32  physical page of logical block j
 *   seq_lens     [B] int32 (device) tokens in each sequence, including the
 *                                   token being decoded; clamped on device to
 *                                   [0, min(max_seq_len, max_blocks*64)]
 *   max_seq_len  host upper bound of seq_lens (sizes the split plan)
 *   B >= 1; H a multiple of 16, 16 <= H <= 128
 *   softmax_scale  > 0, finite
 *   num_splits   0 = automatic (enough splits to occupy every compute unit
 *                of the current device, none shorter than a few pages), else
 *                the number of splits a max_seq_len sequence is cut into (>= 1)
 *   workspace    device buffer of at least mla_decode_lowbit_workspace(...)
 *                bytes (may be NULL when that size is 0)
 *   out          [B][H][512] fp32
 *   lse          [B][H] fp32, natural log; -inf for an empty sequence (whose
 *                out row is 0)
 */
int mla_decode_lowbit(int f, const uint16_t* q_lat, const uint16_t* q_rope,
                      const uint8_t* pages, int64_t num_pages, const uint16_t* prot,
                      int32_t num_seq_slots, const int32_t* seq_slot,
                      const int32_t* block_table, int32_t max_blocks,
                      const int32_t* seq_lens, int32_t max_seq_len, int32_t B,
                      int32_t H, float softmax_scale, int32_t num_splits,
                      void* workspace, size_t workspace_bytes, float* out,
                      float* lse, void* stream);

/*
 * mla_decode_lowbit_append -- one decode step with the fused cache writer in
 * the same launch [QuantMLA App. C.5]: the result equals
 *   kv_quant_append(f, latent, k_rope, slot_mapping, seq_slot, pos, new_len,
 *                   B, pages, num_pages, prot, num_seq_slots)
 * with, for each sequence b of length L = seq_lens[b] >= 1,
 *   pos = L - 1, new_len = L,
 *   slot_mapping = block_table[b][(L-1)/64] * 64 + (L-1) % 64,
 * followed by mla_decode_lowbit(...) with the same remaining arguments --
 * the same page bytes, protection rows, out and lse.  The token at L - 1 is
 * the one being decoded: its packed copy and bf16 protection row are stored
 * for later calls, and this call's attention reads its bf16 row from
 * latent / k_rope directly.
 *
 *   latent [B][512], k_rope [B][64] bf16: the newest token of each sequence
 *   pages, prot: written (token slots and protection rows as above)
 *   other arguments, workspace size and errors: as mla_decode_lowbit.
 * Sequences with L = 0 append nothing; a block-table entry outside
 * [0, num_pages) for block (L-1)/64 stores nothing (that token then reads as
 * an unusable slot, as in mla_decode_lowbit).  A sequence whose seq_lens[b]
 * exceeds min(max_seq_len, max_blocks*64) appends nothing either: its length
 * is clamped as in mla_decode_lowbit, the clamped last token is one the
 * cache already holds, and that sequence's result is exactly
 * mla_decode_lowbit's (pages and prot untouched).
 */
int mla_decode_lowbit_append(int f, const uint16_t* latent, const uint16_t* k_rope,
                             const uint16_t* q_lat, const uint16_t* q_rope, uint8_t* pages,
                             int64_t num_pages, uint16_t* prot, int32_t num_seq_slots,
                             const int32_t* seq_slot, const int32_t* block_table,
                             int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                             int32_t B, int32_t H, float softmax_scale, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, float* out, float* lse,
                             void* stream);

/*
 * mla_decode_lowbit_noalloc -- mla_decode_lowbit for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument, and no
 * allocation by the call.  The split partials go to a scratch array of
 * MLA_LB_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on each GPU
 * it runs on until the process ends.
 *   - Same arguments, result and errors as mla_decode_lowbit, without
 *     workspace / workspace_bytes.
 *   - num_splits = 0: the automatic plan, limited to as many splits as the
 *     scratch holds (B * splits * H * 516 * 4 bytes <= 64 MiB; one split,
 *     which needs no scratch, when not even two fit).  With the same plan the
 *     result is bit-identical to mla_decode_lowbit's.
 *   - num_splits > 0 whose partials exceed the scratch: MLA_LB_EWORKSPACE,
 *     returned on the host before any HIP call.
 *   - The first call on a device looks up that device's scratch address
 *     (hipGetSymbolAddress, a host call that allocates nothing); make it
 *     outside a graph capture.  A failed lookup returns MLA_LB_EHIP.
 *   - Calls on one GPU share its scratch: calls that overlap in time on one
 *     GPU (different streams or host threads) race and give undefined
 *     results.  Serialise them (one stream, or events).
 */
int mla_decode_lowbit_noalloc(int f, const uint16_t* q_lat, const uint16_t* q_rope,
                              const uint8_t* pages, int64_t num_pages, const uint16_t* prot,
                              int32_t num_seq_slots, const int32_t* seq_slot,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t H,
                              float softmax_scale, int32_t num_splits, float* out, float* lse,
                              void* stream);

/*
 * mla_decode_lowbit_mq_workspace -- bytes of workspace mla_decode_lowbit_mq
 * needs for the same (f, B, nq, H, max_seq_len, num_splits) (host; the
 * automatic plan reads the current device as mla_decode_lowbit_workspace).
 *   bytes (host out)
 */
int mla_decode_lowbit_mq_workspace(int f, int32_t B, int32_t nq, int32_t H,
                                   int32_t max_seq_len, int32_t num_splits, size_t* bytes);

/*
 * mla_decode_lowbit_mq -- attention of nq consecutive new tokens per sequence
 * over the mixed-precision cache (several queries per sequence: a verify step
 * of speculative decoding, or the tail of a chunked prefill -- the
 * compute-friendly side of MLA attention [MLA blog §7]).  The nq tokens are
 * the last nq of the sequence and are already in the cache (written by
 * kv_quant_append with new_len = seq_lens[b]).  For L = seq_lens[b], query j
 * (position L - nq + j) attends to its causal prefix [MLA blog §8], tokens
 * [0, L - nq + 1 + j):
 *
 *   S[b,j,h,i] = softmax_scale * (q_lat[b,j,h] . c~_i + q_rope[b,j,h] . k~_R,i)
 *   out[b,j,h] = sum_i softmax_i(S[b,j,h,:]) c~_i,   lse[b,j,h] = ln sum_i e^S
 *
 * with (c~_i, k~_R,i) read as in mla_decode_lowbit for a sequence of length
 * L: the protected set is that of L [QuantMLA §3.3, App. C.5] for every
 * query of the call (the cache holds no other state).  nq = 1 is exactly
 * mla_decode_lowbit.  The nq*H query rows share each reconstructed page: 96,
 * 112, 128 rows and from 176 up run on the 128-row matrix-core kernel (the
 * last block padded), the other counts on 16-row groups.
 *
 *   q_lat  [B][nq][H][512] bf16,  q_rope [B][nq][H][64] bf16
 *   nq >= 1 with nq*H <= MLA_LB_MAX_ROWS (65536 rows: a 512-token prefill
 *          chunk at 128 heads, 4096 tokens at 16); H as in mla_decode_lowbit.
 *          Each 128-row block reconstructs every page it reads, so a chunk of
 *          C tokens at 128 heads costs C page reconstructions per page (vector
 *          work of about a fifth of the block's matrix work)
 *   out    [B][nq][H][512] fp32,  lse [B][nq][H] fp32 (a query whose prefix
 *          is empty, L - nq + 1 + j <= 0, gets out 0 and lse -inf)
 *   workspace: at least mla_decode_lowbit_mq_workspace(...) bytes; a plan
 *          whose workspace would pass 2^60 bytes is refused (MLA_LB_ESHAPE)
 *   other arguments and errors: as mla_decode_lowbit.
 */
int mla_decode_lowbit_mq(int f, const uint16_t* q_lat, const uint16_t* q_rope,
                         const uint8_t* pages, int64_t num_pages, const uint16_t* prot,
                         int32_t num_seq_slots, const int32_t* seq_slot,
                         const int32_t* block_table, int32_t max_blocks,
                         const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t nq,
                         int32_t H, float softmax_scale, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, float* out, float* lse, void* stream);

/*
 * Offline calibration helpers (host, pure; no GPU).  The cache transforms
 * they serve are folded into the model's projections before serving, so the
 * decode path runs unchanged [QuantMLA App. C.1, C.2, D.2]: a content channel
 * j is cached as x_j * s_j with queries and the aggregated latent compensated
 * by 1/s_j; a RoPE frequency pair (2i, 2i+1) shares one scale, with the
 * reciprocal on the query, which keeps every positional score and commutes
 * with the positional rotation.
 *
 * mla_lb_channel_stat -- per channel j < n, the pct-th percentile of |x[r][j]|
 *   over rows r < rows (linear interpolation between order statistics),
 *   x host bf16 [rows][n], stat host fp32 [n].  pct in [0, 100].
 * mla_lb_smooth_scales -- s_j = max(a_j, 1e-8)^(-alpha) from statistics
 *   stat[n] (host fp32); pair_tied != 0 gives channels 2i and 2i+1 the
 *   statistic max(a~_2i, a~_2i+1) (n even).  alpha >= 0; alpha = 0 gives 1.
 *   The candidate rule is read as the SmoothQuant smoothing factor with
 *   activation statistics only (the formula is missing from the pages'
 *   extracted text); alpha is chosen by held-out attention-output error.
 */
int mla_lb_channel_stat(const uint16_t* x, int64_t rows, int32_t n, double pct, float* stat);
int mla_lb_smooth_scales(const float* stat, int32_t n, float alpha, int32_t pair_tied,
                         float* scales);

/*
 * mla_lb_hadamard_rows -- y[r] = x[r] . H_n for r < rows (host, pure), with
 * H_n the normalized Hadamard matrix of order n (Sylvester's +-1 matrix
 * divided by sqrt(n); symmetric and orthogonal, so H_n is its own inverse).
 * The content-path rotation [QuantMLA §3.1, App. C.1] in its fixed form, the
 * deterministic normalized Hadamard of the QuaRot-style baseline
 * [QuantMLA App. D.2]: the latent is cached as c.H (folded into the
 * projection that produces it), the absorbed content query becomes q.H, and
 * the aggregated latent o' maps back as o'.H -- attention is unchanged in
 * exact arithmetic, and each token's outlier channels are spread over all
 * groups before quantization.  Computed in fp64 (fast Walsh-Hadamard
 * butterflies), rounded once to fp32.
 *   x, y  host fp32 [rows][n] (may be the same buffer); n a power of two,
 *   n <= 2^20; rows >= 1.
 */
int mla_lb_hadamard_rows(const float* x, int64_t rows, int32_t n, float* y);

/*
 * mla_lb_dequant_dump -- write the bf16 rows the decode kernel reconstructs
 * for every slot of one page, [64][576] = [c^ | k^_R], using the same device
 * code as mla_decode_lowbit.  For checking the reconstruction bit for bit.
 *   page_id in [0, num_pages)
 */
int mla_lb_dequant_dump(int f, const uint8_t* pages, int64_t num_pages,
                        int64_t page_id, uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_LOWBIT_H */
