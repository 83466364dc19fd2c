/*
 * fa.h -- C ABI of libfa_mi355x: tiled exact attention (forward and backward)
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every batch index b and head h, with N queries and N
 * keys of head dimension d:
 *
 *   S = scale * Q K^T, with S_ij = -inf where key j is not visible to query i,
 *   LSE_i = log sum_j exp(S_ij)              (natural logarithm),
 *   O = exp(S - LSE) V.
 *
 * This is the attention of "02 -- FlashAttention como una optimizacion de
 * roofline" (lynx-cortex), section "El algoritmo naive de attention", computed
 * block by block with the running row maximum and row sum of the online
 * softmax ("El algoritmo Flash (forward)" there; "como funciona" in the
 * tonho.wtf digest) so that no N x N matrix is written to memory.  The
 * backward recomputes the probabilities from Q, K and the saved LSE instead of
 * storing them ("Passo para tras: recalcular em vez de armazenar", the
 * marketmaker.cc article) and uses D_i = dO_i . O_i for the softmax gradient
 * ("como funciona", tonho.wtf digest).
 *
 * Visibility of key j to query i:
 *   [causal == 0 or j <= i]   (future keys excluded -- the causal-mask section
 *                              of the marketmaker.cc article)
 *   and [window == 0 or |i - j| < window]
 *                             (sliding window -- the practice problems of the
 *                              lynx-cortex page; with causal, the window most
 *                              recent keys i - window + 1 .. i)
 *   and [block_mask == NULL or block_mask[i / mask_block][j / mask_block] != 0]
 *                             (block-sparse attention -- block-sparse paragraph
 *                              of the agihunt.info summary of the paper).
 * A query row with no visible key gets O = 0, LSE = -inf and contributes
 * nothing to the gradients.
 *
 * Grouped K/V heads (multi-query and grouped-query attention, sections 4-6 of
 * "Atencao Eficiente em Escala", living-dl-book): K and V may have H_kv heads,
 * H_kv dividing H; query head h reads K/V head h / (H / H_kv), and dK, dV of a
 * K/V head are the sums over the H / H_kv query heads that read it.
 *
 * Dropout (applied inside the fused kernels and regenerated in the backward
 * from the generator state instead of being stored -- "como funciona" in the
 * tonho.wtf digest; the algorithm paragraph of the agihunt.info summary).
 * With t = floor(256 * dropout_p): for query i, key j of query head
 * b * H + h, one Philox4x32-10 evaluation (Salmon et al., "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC 2011) with counter
 * (j / 4, i / 4, b * H + h, offset) and key (seed mod 2^32, seed / 2^32)
 * gives four 32-bit words; the weight P_ij is kept iff byte (j mod 4) of word
 * (i mod 4) is >= t, and kept weights are multiplied by 256 / (256 - t):
 *   O = (P o Z) V with LSE the normaliser of P (not of P o Z),
 *   dP = Z o (dO V^T), D_i = dO_i . O_i, dS = P o (dP - D).
 * The drop probability actually used is t / 256.
 *
 * Layouts.  Q, O, dO, dQ are contiguous row-major tensors of shape
 * (B, H, N, d) in the problem's dtype; element (b, h, n, c) sits at
 * ((b * H + h) * N + n) * d + c.  K, V, dK, dV are (B, H_kv, N, d) in the same
 * way.  LSE is float32 (B, H, N).  block_mask is
 * uint8 [N / mask_block][N / mask_block], row = query block, shared by all
 * (b, h).  Every tensor pointer is a DEVICE pointer (hipMalloc'd or equivalent)
 * unless stated otherwise; device pointers must be 16-byte aligned.
 *
 * Streams.  `stream` is the HIP stream to enqueue on (NULL = the default
 * stream).  All work is enqueued asynchronously on it; no call synchronises
 * the host.
 *
 * Ownership.  The caller allocates and owns every buffer, including the
 * workspace, and keeps them alive until the enqueued work has completed.  The
 * library allocates nothing, keeps no state between calls and is thread-safe.
 *
 * Errors.  Every entry point returns FA_OK (0) on success or a negative status
 * before anything is enqueued.  There is never a silent fallback to another
 * implementation: an unsupported problem is an error.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_dtype {
  FA_F32 = 0,  /* float32 in, float32 arithmetic (vector ALU path)          */
  FA_F16 = 1,  /* float16 in/out, float32 accumulation on matrix cores       */
  FA_BF16 = 2  /* bfloat16 in/out, float32 accumulation on matrix cores      */
};

enum fa_status {
  FA_OK = 0,
  FA_ERR_ARG = -1,          /* null pointer, non-positive size, scale not finite
                               and positive, misaligned pointer, negative
                               window, H_kv not dividing H, dropout_p outside
                               [0, 1), an unknown flag bit                     */
  FA_ERR_UNSUPPORTED = -2,  /* d not in {64, 128}; unknown dtype; a block mask
                               whose block is not a positive multiple of 128 or
                               does not divide N                               */
  FA_ERR_WORKSPACE = -3,    /* workspace missing, smaller than required, or not
                               16-byte aligned (every entry point that takes
                               one)                                            */
  FA_ERR_LAUNCH = -4,       /* the HIP runtime rejected a kernel launch, or a
                               HIP query needed to set up the call failed      */
  FA_ERR_SCRATCH = -5       /* the problem needs more scratch than the static
                               buffer of fa_fwd_decode_noalloc holds           */
};

typedef struct fa_problem {
  int32_t B, H, N, d;         /* batch, query heads, sequence length, head dim */
  int32_t dtype;              /* enum fa_dtype                                 */
  int32_t causal;             /* 0 or 1                                        */
  float scale;                /* multiplies Q K^T, e.g. 1/sqrt(d); finite, > 0 */
  const uint8_t* block_mask;  /* device pointer or NULL (dense)                */
  int32_t mask_block;         /* side of one mask block; used iff block_mask   */
  int32_t window;             /* 0: no window; W > 0: |i - j| < W              */
  int32_t H_kv;               /* heads of K and V; 0 means H; must divide H    */
  float dropout_p;            /* in [0, 1); 0 disables dropout                 */
  uint64_t seed;              /* dropout generator key                         */
  uint32_t offset;            /* dropout counter word: one value per call that
                                 must draw a fresh mask with the same seed     */
  uint32_t flags;             /* 0, or FA_REUSE_LISTS | FA_BWD_ATOMIC_DQ       */
} fa_problem;

/* fa_problem.flags bits.
 * FA_REUSE_LISTS: the workspace passed to this call already holds the block
 *   lists compiled for this problem's block_mask, N and mask_block -- written
 *   by an earlier fa_fwd, fa_bwd or fa_bwd_dq call on the same buffer -- so
 *   this call skips compiling them.  The lists sit at the start of both the
 *   forward and the backward workspace, so a caller that gives the forward
 *   and the backward of one step the same buffer (of fa_workspace_size(p, 1)
 *   bytes) compiles the mask once per step.  The library cannot check the
 *   contents: with lists of another mask, or none, the behaviour is undefined
 *   (wrong results, or reads outside the workspace).  Ignored without a
 *   block mask and for FA_F32 (which reads the mask itself). */
#define FA_REUSE_LISTS 1u

/* FA_BWD_ATOMIC_DQ: fa_bwd runs the single-pass backward of the pages'
 *   backward loop ("Passo para tras: recalcular em vez de armazenar",
 *   marketmaker.cc article): the key-outer kernel also forms dQ += dS K for its
 *   keys and adds it into a float32 accumulator (B,H,N,d) in the workspace with
 *   atomic adds, so S and dP are computed once per visible pair (10 d FLOPs)
 *   instead of in two kernels (14 d).  dq then depends on the order of the
 *   adds: repeated calls can differ in the last bits (dk and dv do not).
 *   FA_F16 and FA_BF16 only (FA_F32: FA_ERR_UNSUPPORTED).  fa_bwd_dq and
 *   fa_bwd_dkdv, the stages of the two-kernel backward, return FA_ERR_ARG with
 *   this flag; the forward entry points ignore it. */
#define FA_BWD_ATOMIC_DQ 2u

/* Bytes of device workspace that fa_fwd (pass 0) or fa_bwd (pass 1) needs for
 * problem p; 0 if none.  Host-only arithmetic, no GPU call.  Returns 0 for an
 * invalid problem (the entry point itself then reports the error).  Layout:
 * with a block mask (FA_F16, FA_BF16) the compiled block lists come first in
 * both passes; the backward then holds D (float32, B*H*N) on the next
 * 256-byte boundary and, with FA_BWD_ATOMIC_DQ (FA_F16, FA_BF16), the float32
 * dQ accumulator (B*H*N*d) on the next.  The backward's size is never
 * smaller than the forward's, so one buffer of the backward's size serves
 * both. */
size_t fa_workspace_size(const fa_problem* p, int pass);

/* Forward.  Reads q, k, v; overwrites o (B,H,N,d, dtype) and lse (B,H,N,
 * float32, natural log).  workspace: device buffer of at least
 * fa_workspace_size(p, 0) bytes (may be NULL when that is 0). */
int fa_fwd(const fa_problem* p, const void* q, const void* k, const void* v, void* o,
           float* lse, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Backward of f = <O, dO>.  Reads q, k, v, o, dout and lse, which must be the
 * O and LSE that fa_fwd produced for the same q, k, v and problem (with
 * dropout: the same seed and offset, so the same mask is regenerated).
 * Overwrites (does not accumulate into) dq, dk, dv.  workspace: at least
 * fa_workspace_size(p, 1) bytes; it receives D_i = dO_i . O_i (float32, B*H*N)
 * and, with a block mask, the compiled block lists (unless FA_REUSE_LISTS
 * says they are there already); with FA_BWD_ATOMIC_DQ also the float32 dQ
 * accumulator. */
int fa_bwd(const fa_problem* p, const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
           size_t ws_bytes, hipStream_t stream);

/* The two stages of fa_bwd, for callers that schedule or time them apart.
 * fa_bwd_dq: computes D_i = dO_i . O_i into the workspace (and, with a block
 *   mask, the compiled block lists), then writes dq.
 * fa_bwd_dkdv: writes dk and dv; reads D (and the lists) from the SAME
 *   workspace, so it must be enqueued after fa_bwd_dq on the same stream with
 *   unchanged arguments.  fa_bwd is exactly fa_bwd_dq followed by fa_bwd_dkdv.
 * Arguments, layouts and errors are those of fa_bwd. */
int fa_bwd_dq(const fa_problem* p, const void* q, const void* k, const void* v, const void* o,
              const void* dout, const float* lse, void* dq, void* workspace, size_t ws_bytes,
              hipStream_t stream);
int fa_bwd_dkdv(const fa_problem* p, const void* q, const void* k, const void* v,
                const void* dout, const float* lse, void* dk, void* dv, void* workspace,
                size_t ws_bytes, hipStream_t stream);

/* Block-mask compilation (the step both passes run first when a block mask is
 * given).  mask: device uint8 [nb][nb]; writes, all int32 device arrays:
 *   row_ptr[nb + 1], col_idx[nnz]: for query block r, the kept key blocks
 *     col_idx[row_ptr[r] .. row_ptr[r+1]) in increasing order;
 *   col_ptr[nb + 1], row_idx[nnz]: for key block c, the query blocks that keep
 *     it, row_idx[col_ptr[c] .. col_ptr[c+1]) in increasing order.
 * col_idx and row_idx must hold nb*nb entries (the worst case). */
int fa_mask_compile(const uint8_t* mask, int32_t nb, int32_t* row_ptr, int32_t* col_idx,
                    int32_t* col_ptr, int32_t* row_idx, hipStream_t stream);

/* Decode-shaped forward (a few queries against many keys, with grouped K/V
 * heads).  q and o are (B, H, n_q, d) in the
 * problem's dtype, lse is float32 (B, H, n_q); k and v are (B, H_kv, N, d) with
 * N = p->N.  Query i of each head sits at position N - n_q + i of the key
 * sequence, and causal / window visibility use that position (with causal and
 * n_q = 1 the query sees every key).  The result is the attention defined at
 * the top of this file restricted to those rows.  Inside, the key range is cut
 * into splits computed by separate workgroups, each leaving the running
 * maximum / running sum result of its keys (O_s normalised, LSE_s), and a
 * second kernel merges them with LSE = log sum_s exp(LSE_s),
 * O = sum_s exp(LSE_s - LSE) O_s -- the merge step of the online softmax
 * ("A recorrencia do softmax online", marketmaker.cc article).
 * Requirements: 1 <= n_q <= N; dtype FA_F16 or FA_BF16 (FA_F32 ->
 * FA_ERR_UNSUPPORTED); block_mask == NULL and dropout_p == 0 (else
 * FA_ERR_UNSUPPORTED); the other fields as for fa_fwd.  workspace: at least
 * fa_decode_workspace_size(p, n_q) bytes (float32 partial results; may be NULL
 * when that is 0).  The split count depends only on the problem. */
size_t fa_decode_workspace_size(const fa_problem* p, int32_t n_q);
int fa_fwd_decode(const fa_problem* p, int32_t n_q, const void* q, const void* k, const void* v,
                  void* o, float* lse, void* workspace, size_t ws_bytes, hipStream_t stream);

/* fa_fwd_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as fa_fwd_decode, without the workspace:
 * the float32 split partials live in a static device buffer inside the
 * library, 64 MiB (67108864 bytes) per GPU, held from the first call on that
 * GPU until the process ends.  A problem whose fa_decode_workspace_size
 * exceeds 64 MiB returns FA_ERR_SCRATCH before anything is enqueued (e.g.
 * d = 128 with more than 63 query rows per K/V head, rows = H / H_kv * n_q).
 * The call allocates nothing and clears nothing (every partial the merge
 * reads is written first in the same call).  `stream` must belong to the
 * current device (else FA_ERR_ARG).  All calls on one GPU share that GPU's
 * buffer: calls whose work overlaps on one GPU (other streams, other host
 * threads) race on it and must be ordered by the caller, e.g. by issuing
 * them on one stream. */
int fa_fwd_decode_noalloc(const fa_problem* p, int32_t n_q, const void* q, const void* k,
                          const void* v, void* o, float* lse, hipStream_t stream);

/* FP8 forward: block quantisation with a random Hadamard-style rotation
 * ("Atencao Eficiente em Escala", section 10 on FlashAttention-3: Q, K, V are
 * quantised to FP8 with one scale per tile after an orthogonal randomised
 * Hadamard projection that spreads outlier coordinates; the rotation is undone
 * after the product).  Two calls:
 *
 * fa_fp8_quantize rotates every row of q, k, v by M = diag(signs) H / sqrt(d)
 * (H the d x d Sylvester Hadamard matrix; float32 butterflies with pair
 * distances 1, 2, ..., d/2, then a multiply by float32(1 / sqrt(d))), and
 * quantises each block of 64 rows of one head to E4M3 (bias 7, largest finite
 * value 448, round to nearest even) with the scale 2^e, e the smallest integer
 * with max |row value| <= 448 * 2^e.  Rows past N (up to N64 = N rounded up to
 * a multiple of 64) are zero.  Results go to the workspace:
 *   Q codes  uint8 (B H, N64, d) row-major;  K codes uint8 (B H_kv, N64, d);
 *   V codes  uint8 (B H_kv, N64 / 64, d, 64): per 64-key tile, row c holds
 *            column c of V, byte p holding key 32 (i / 16) + 8 ((i % 16) / 4)
 *            + 4 h + i % 4 of the tile, h = p / 32, i = p % 32;
 *   then int8 exponents e of Q (B H, N64 / 64), K and V (B H_kv, N64 / 64);
 *   each of the six regions starts on a 256-byte boundary, in that order.
 * fa_fwd_fp8 computes attention on those codes: S = scale Qr Kr^T on the FP8
 * matrix cores with the block scales applied inside the product, the online
 * softmax in float32, probabilities (at most 256) rounded to E4M3 for the P V
 * product, float32 accumulation, and O = (P Vr / l) M^T written in the
 * problem's dtype (B, H, N, d), with lse float32 (B, H, N) the natural-log
 * LSE of the scores.  Masks: causal and window as for fa_fwd.
 *
 * signs: device float32[d], each +1 or -1 (the caller's random draw; the
 * library reads, never writes it).  q, k, v as for fa_fwd.  Requirements:
 * dtype FA_F16 or FA_BF16, block_mask == NULL and dropout_p == 0 (else
 * FA_ERR_UNSUPPORTED); workspace at least fa_fp8_workspace_size(p) bytes,
 * 16-byte aligned (else FA_ERR_WORKSPACE), owned by the caller and left
 * unchanged by fa_fwd_fp8, which reads the codes fa_fp8_quantize left there
 * for the same problem and signs.  fa_fp8_workspace_size returns 0 for a
 * problem the FP8 path does not take. */
size_t fa_fp8_workspace_size(const fa_problem* p);
int fa_fp8_quantize(const fa_problem* p, const float* signs, const void* q, const void* k,
                    const void* v, void* workspace, size_t ws_bytes, hipStream_t stream);
int fa_fwd_fp8(const fa_problem* p, const float* signs, const void* workspace, size_t ws_bytes,
               void* o, float* lse, hipStream_t stream);

/* Static string for a status code. */
const char* fa_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
