/*
 * dsa.h - C ABI of libdsa.so: forward hot path of a gated DSA layer on MI355X (gfx950).
 *
 * The path (NeMo AutoModel "Kimi-K3.1-Pro" model-coverage page, summary and Implementation
 * Limits; archdiff.com "Kimi K3.1 Pro" blueprint; kimi_k3 API index, KimiK3TextConfig):
 *   1. LayerNorm on the indexer key k_I (blueprint component list: the indexer key is layer-normed).
 *   2. Indexer scores S(t,s) = sum_h w[t,h] * ReLU(q_I[t,h,:] . LN(k_I)[s,:]) over every causal
 *      key s of token t, bf16 operands with FP32 accumulation (Implementation Limits, 2nd bullet).
 *      The T x T score matrix is never stored. The scoring form and the tie rule below are the
 *      problem statement's; the pages only name a fused indexer.
 *   3. Hard top-k (k <= 2048) per query, ties to the lower key index; a token with at most k
 *      causal keys keeps all of them (summary; Implementation Limits, 3rd and 4th bullets).
 *   4. Sparse latent attention over the selected rows of the latent KV (kv_lora_rank 512 plus
 *      64 unrotated dims, no positional encoding), softmax in FP32 (Implementation Limits, 1st
 *      and 2nd bullets; blueprint tagline; API index mla_use_nope).
 *   5. Per-head V up-projection 512 -> 128 (the effective kv_b_proj V weight) and the sigmoid
 *      output gate out = sigma(g) * o (paragraph on the output gate and kv_b_proj; blueprint
 *      output-gate component).
 *
 * Conventions for every entry point
 *  - bf16 tensors are passed as bf16 bit patterns (uint16_t) in device memory, row-major,
 *    contiguous, 16-byte aligned (k_I, w and gate: 2-byte aligned suffices). Integer tensors are
 *    int32 in device memory: topk_idx is written with 16-byte stores and must be 16-byte aligned
 *    where an entry point writes it, 4-byte aligned where it is only read. float32 tensors are
 *    4-byte aligned.
 *  - Token axis: keys and key-side tensors (k_I, kv) cover all T tokens. Query-side tensors
 *    (q_I, w, q, gate) and outputs (topk_idx, out, lse) cover only the rows
 *    [q_begin, q_end) of the shape, indexed from 0 (local row r is global token q_begin + r).
 *  - Packed documents are contiguous (model-coverage page: interior holes are not supported);
 *    cu_seqlens gives their boundaries. A token's causal keys are the tokens of its own
 *    document up to and including itself.
 *  - The caller owns every buffer. The library never allocates, frees or synchronises; work is
 *    enqueued on the given HIP stream (a hipStream_t passed as void*, NULL = default stream).
 *  - Argument checks run on the host before any HIP call and return a status; nothing is
 *    enqueued when a check fails. A failed launch returns DSA_ERR_LAUNCH. Faults inside kernels
 *    surface at the caller's next synchronisation. No C++ exception crosses this ABI.
 *  - Calls that share a workspace must not overlap.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer, bad cu_seqlens */
  DSA_ERR_UNSUPPORTED = 2, /* shape outside the supported set, or a device that can hold more
                              indexer workgroups at once than the workspace has candidate slots */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than dsa_workspace_size() */
  DSA_ERR_LAUNCH = 4,      /* a kernel launch failed */
  DSA_ERR_TOO_LARGE = 5    /* beyond the fixed scratch of dsa_index_topk_noalloc */
} dsa_status;

/* Shapes of one call. Supported: (H_I, d_I) in {(64,128), (4,64)}; H in {96, 16};
 * 1 <= topk <= 2048. Latent rows are 576 wide (512 V dims + 64 key-only dims); the head output
 * is 128 wide. */
typedef struct dsa_shape {
  int32_t T;                      /* tokens (keys) over all packed documents, >= 1 */
  int32_t n_docs;                 /* >= 1 */
  const int32_t* cu_seqlens_host; /* [n_docs+1] host memory: 0 = c0 < c1 < ... < c_n = T;
                                     may be NULL only when n_docs == 1 */
  const int32_t* cu_seqlens_dev;  /* the same values in device memory; NULL only when n_docs == 1 */
  int32_t q_begin;                /* first query row processed, 0 <= q_begin < q_end */
  int32_t q_end;                  /* one past the last query row; 0 means T */
  int32_t topk;                   /* k */
  int32_t H_I;                    /* indexer heads */
  int32_t d_I;                    /* indexer head dim */
  int32_t H;                      /* attention heads */
  float ln_eps;                   /* LayerNorm eps on the indexer key (> 0), e.g. 1e-5 */
  float softmax_scale;            /* logit scale (> 0), e.g. 1/sqrt(192) */
} dsa_shape;

/* Bytes of device workspace the entry points need for this shape (256-byte aligned start
 * required). Returns 0 if the shape is invalid or unsupported. Pure host function. */
size_t dsa_workspace_size(const dsa_shape* shape);

/* Host-only argument check of a shape (no HIP call): DSA_OK, DSA_ERR_INVALID_ARG or
 * DSA_ERR_UNSUPPORTED. Every entry point runs it first. */
dsa_status dsa_check_shape(const dsa_shape* shape);

/* Steps 1-3. Inputs: q_I [rows, H_I, d_I] bf16; k_I [T, d_I] bf16; ln_gamma, ln_beta [d_I]
 * float32 device arrays or NULL (identity); w [rows, H_I] bf16 (any sign).
 * Output: topk_idx [rows, topk] int32. Row r holds min(topk, n) distinct global token indices of
 * its causal keys (n = number of causal keys), in ascending order, then -1 up to topk.
 * Workspace: >= dsa_workspace_size(shape) bytes (holds LN(k_I), and the candidate token indices of
 * the rows being selected in 256 fixed slots, one per indexer workgroup in flight). */
dsa_status dsa_index_topk(const dsa_shape* shape, const uint16_t* q_I, const uint16_t* k_I,
                          const float* ln_gamma, const float* ln_beta, const uint16_t* w,
                          int32_t* topk_idx, void* workspace, size_t workspace_bytes, void* stream);

/* Steps 1-3 with the FP8 indexer, the alternative the model-coverage page sets beside its BF16
 * one (Implementation Limits, 2nd bullet: the BF16 indexer is not the FP8 indexer of some serving
 * kernels). The pages give no recipe; this one: each 128-value row (LN(k_I) of a key, one head of
 * q_I) is scaled by a power of two 2^-e, e the smallest integer with max|row| * 2^-e <= 448, and
 * rounded to OCP E4M3 (nearest, ties to even); scores are
 *   S(t,s) = 2^e_k[s] * sum_h (w[t,h] * 2^e_q[t,h]) * ReLU(sum_i q8[t,h,i] * k8[s,i])
 * with exact products and FP32 sums; top-k and its tie rule as in dsa_index_topk. Supported for
 * (H_I, d_I) = (64, 128) only (else DSA_ERR_UNSUPPORTED). Same arguments and workspace as
 * dsa_index_topk; the workspace also holds the E4M3 operands. */
dsa_status dsa_index_topk_fp8(const dsa_shape* shape, const uint16_t* q_I, const uint16_t* k_I,
                              const float* ln_gamma, const float* ln_beta, const uint16_t* w,
                              int32_t* topk_idx, void* workspace, size_t workspace_bytes, void* stream);

/* Steps 1-3 with the key LayerNorm fused into the indexer's key-chunk loads (archdiff "Kimi K3.1
 * Pro" blueprint: LayerNorm on the indexer key; model-coverage page, Implementation Limits, 2nd
 * bullet: one fused indexer). Each workgroup normalises the raw k_I rows of every chunk it stages, in
 * double with one rounding to bf16, so LN(k_I) is never written; the results are identical to
 * dsa_index_topk's. It normalises each key once per workgroup that stages it (about T/16 times), so
 * it is the slower form; dsa_index_topk normalises each key once. Same arguments and workspace as
 * dsa_index_topk, except that k_I must be 16-byte aligned; (H_I, d_I) = (64, 128) only (else
 * DSA_ERR_UNSUPPORTED). */
dsa_status dsa_index_topk_fused_ln(const dsa_shape* shape, const uint16_t* q_I, const uint16_t* k_I,
                                   const float* ln_gamma, const float* ln_beta, const uint16_t* w,
                                   int32_t* topk_idx, void* workspace, size_t workspace_bytes, void* stream);

/* The FP8 indexer's operand quantisation on its own: n_rows rows of 128 bf16 values (x, 16-byte
 * aligned) -> q8 [n_rows, 128] E4M3 codes (16-byte aligned) and scale [n_rows] float32, the row's
 * power of two 2^e as above. No workspace. */
dsa_status dsa_quantize_fp8(int64_t n_rows, const uint16_t* x, uint8_t* q8, float* scale, void* stream);

/* Steps 1-3 without a workspace and without allocating device memory, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same inputs, output and results as dsa_index_topk. The scratch it needs instead of the workspace
 * is a fixed 110,134,272-byte device array per GPU, held from the first call on that GPU until the
 * process ends; it limits the shape to T <= 131072 and at most 64 documents (else
 * DSA_ERR_TOO_LARGE, checked on the host before any HIP call). Every call on a GPU uses that GPU's
 * one array and leaves its contents behind (each call clears what must start at zero itself):
 * calls that overlap on one GPU, on any streams, race and must not be made. */
dsa_status dsa_index_topk_noalloc(const dsa_shape* shape, const uint16_t* q_I, const uint16_t* k_I,
                                  const float* ln_gamma, const float* ln_beta, const uint16_t* w,
                                  int32_t* topk_idx, void* stream);

/* Steps 4-5 for caller-supplied indices. Inputs: q [rows, H, 576] bf16 (already absorbed into
 * the latent space; dims 0..511 pair with the compressed KV, 512..575 with the key-only dims);
 * kv [T, 576] bf16; topk_idx [rows, topk] int32 (entries outside [0, T) are ignored; a row with
 * no usable entry yields zeros and lse = -inf); W_UV [H, 512, 128] bf16; gate [rows, H] bf16
 * gate logits. Outputs: out [rows, H, 128] bf16 = bf16(sigmoid(gate) * o);
 * lse [rows, H] float32 natural-log softmax normaliser, or NULL. Only the first min(topk, n)
 * entries of a row are read (n = the row's number of causal keys); every usable one among them
 * is attended, duplicates included; causality of the indices is the caller's contract.
 * Workspace: >= dsa_workspace_size(shape) bytes (holds o_lat for up to 2048 rows at a time). */
dsa_status dsa_sparse_mla_fwd(const dsa_shape* shape, const uint16_t* q, const uint16_t* kv,
                              const int32_t* topk_idx, const uint16_t* W_UV, const uint16_t* gate,
                              uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Step 4 alone: sparse latent attention into a caller buffer. Inputs as dsa_sparse_mla_fwd.
 * Output: o_lat [rows, H, 512] bf16 = softmax-weighted sum of the V parts (dims 0..511) of the
 * selected latent rows, before the up-projection; lse as in dsa_sparse_mla_fwd. No workspace. */
dsa_status dsa_sparse_attention_latent(const dsa_shape* shape, const uint16_t* q, const uint16_t* kv,
                                       const int32_t* topk_idx, uint16_t* o_lat, float* lse, void* stream);

/* Step 5 alone: out [rows, H, 128] bf16 = bf16(sigmoid(gate) * (o_lat . W_UV[h])) per head, from
 * o_lat [rows, H, 512] bf16, W_UV [H, 512, 128] bf16 and gate [rows, H] bf16. No workspace. */
dsa_status dsa_up_gate(const dsa_shape* shape, const uint16_t* o_lat, const uint16_t* W_UV, const uint16_t* gate,
                       uint16_t* out, void* stream);

/* Variants of steps 4-5 (archdiff.com "Kimi K3.1 Pro" blueprint, entry "Output gate + sink":
 * sigma(x W_g) * o with a learnable sink). A NULL variant pointer means the defaults: gate
 * [rows, H] and no sink. */
typedef struct dsa_mla_variant {
  int32_t gate_per_dim;   /* 0: gate [rows, H], one logit per (row, head), broadcast over the 128
                             outputs; 1: gate [rows, H, 128], one logit per output element
                             (16-byte aligned) */
  const float* sink;      /* [H] float32 device array of per-head sink logits, in the units of the
                             scaled logits (natural log), or NULL. Head h's softmax denominator gains
                             exp(sink[h]), a logit whose value row is zero: the keys' weights then sum
                             to 1 - exp(sink[h] - lse), and lse includes the sink. */
} dsa_mla_variant;

/* dsa_sparse_attention_latent with a variant: only its sink changes o_lat and lse (the gate is not
 * applied here). NULL: identical to dsa_sparse_attention_latent. No workspace. */
dsa_status dsa_sparse_attention_latent_ex(const dsa_shape* shape, const dsa_mla_variant* variant, const uint16_t* q,
                                          const uint16_t* kv, const int32_t* topk_idx, uint16_t* o_lat, float* lse,
                                          void* stream);

/* dsa_sparse_mla_fwd with a variant (NULL: identical to dsa_sparse_mla_fwd). */
dsa_status dsa_sparse_mla_fwd_ex(const dsa_shape* shape, const dsa_mla_variant* variant, const uint16_t* q,
                                 const uint16_t* kv, const int32_t* topk_idx, const uint16_t* W_UV,
                                 const uint16_t* gate, uint16_t* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Steps 1-5 in one call: the union of the two argument lists; topk_idx is written and then used. */
dsa_status dsa_fused_fwd(const dsa_shape* shape, const uint16_t* q_I, const uint16_t* k_I,
                         const float* ln_gamma, const float* ln_beta, const uint16_t* w,
                         const uint16_t* q, const uint16_t* kv, const uint16_t* W_UV,
                         const uint16_t* gate, int32_t* topk_idx, uint16_t* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/* dsa_fused_fwd with a variant of steps 4-5 (NULL: identical to dsa_fused_fwd). */
dsa_status dsa_fused_fwd_ex(const dsa_shape* shape, const dsa_mla_variant* variant, const uint16_t* q_I,
                            const uint16_t* k_I, const float* ln_gamma, const float* ln_beta, const uint16_t* w,
                            const uint16_t* q, const uint16_t* kv, const uint16_t* W_UV, const uint16_t* gate,
                            int32_t* topk_idx, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream);

/* The step before sparse MLA: the per-head W_UK absorption that gives the latent query (model-coverage
 * page, Implementation Limits, 2nd bullet: sparse MLA never expands the per-head keys;
 * KimiK3TextConfig: qk_nope_head_dim 128, kv_lora_rank 512, qk_rope_head_dim 64, mla_use_nope).
 * W_UK [H, 512, 128] bf16 is the key half of the kv_b_proj effective weight (head h's expanded key
 * of a token is k_nope[d] = sum_c c_KV[c] * W_UK[h,c,d]). Inputs q_nope [rows, H, 128] and q_pe
 * [rows, H, 64] bf16; output q [rows, H, 576] bf16 with
 *   q[t,h,c] = bf16(sum_d q_nope[t,h,d] * W_UK[h,c,d]) for c < 512 (FP32 accumulation), and
 *   q[t,h,512 + j] = q_pe[t,h,j] (unrotated),
 * the q that dsa_sparse_mla_fwd and dsa_fused_fwd take. Rows as in dsa_shape; no workspace. */
dsa_status dsa_q_absorb(const dsa_shape* shape, const uint16_t* q_nope, const uint16_t* q_pe,
                        const uint16_t* W_UK, uint16_t* q, void* stream);

/* The step after the gate: the attention output projection o_proj (model-coverage page, paragraph
 * on the output gate; KimiK3TextConfig hidden_size 7168). x [rows, H * 128] bf16 is the out of the
 * path (the gated head outputs of a row, heads in order); W_o [d_model, H * 128] bf16 in the
 * [out_features, in_features] layout; y [rows, d_model] bf16 = bf16(x W_o^T), FP32 accumulation.
 * d_model must be a positive multiple of 256 (else DSA_ERR_UNSUPPORTED). Rows as in dsa_shape;
 * no workspace. */
dsa_status dsa_o_proj(const dsa_shape* shape, const uint16_t* x, const uint16_t* W_o, int32_t d_model,
                      uint16_t* y, void* stream);

/* Backward of steps 4-5 on the native 96 heads (model-coverage page, paragraph after the
 * Implementation Limits bullets: the backward runs 96 heads without padding; 3rd bullet: hard top-k
 * carries no gradient, so topk_idx is a constant and the indexer has no backward). For the loss
 * L = sum(dout * out) of dsa_sparse_mla_fwd (per-head gate, no sink) on the same q, kv, topk_idx,
 * W_UV and gate, given that call's out [rows, H, 128] and lse [rows, H]:
 *   dq [rows, H, 576], dkv [T, 576], dW_UV [H, 512, 128], dgate [rows, H], all float32.
 * dkv and dW_UV are overwritten (zeroed, then accumulated over the rows in an order that atomic
 * operations decide, so their last bits may differ from call to call); dq and dgate are written.
 * H must be 96 (else DSA_ERR_UNSUPPORTED). Workspace: >= dsa_bwd_workspace_size(shape) bytes. */
size_t dsa_bwd_workspace_size(const dsa_shape* shape);
dsa_status dsa_sparse_mla_bwd(const dsa_shape* shape, const uint16_t* q, const uint16_t* kv,
                              const int32_t* topk_idx, const uint16_t* W_UV, const uint16_t* gate,
                              const uint16_t* out, const float* lse, const uint16_t* dout, float* dq,
                              float* dkv, float* dW_UV, float* dgate, void* workspace,
                              size_t workspace_bytes, void* stream);

/* The same backward for the gate and sink variants of dsa_sparse_mla_fwd_ex (archdiff.com blueprint,
 * "Output gate + sink"), given that call's out and lse (which includes the sink):
 *   - variant->gate_per_dim = 1: gate [rows, H, 128] (16-byte aligned) and dgate [rows, H, 128]
 *     (16-byte aligned), dgate = (1 - sigmoid(gate)) * dout * out element by element;
 *   - variant->sink [H]: dsink [H] float32 receives dL/dsink[h] = -sum over rows of
 *     exp(sink[h] - lse) * sum_d dout * out (the sink is a softmax logit with a zero value row);
 *     dsink must be NULL without a sink and non-NULL with one (else DSA_ERR_INVALID_ARG).
 * A NULL variant is dsa_sparse_mla_bwd. dsink is overwritten (summed over the rows in a fixed
 * order). Workspace as dsa_sparse_mla_bwd. */
dsa_status dsa_sparse_mla_bwd_ex(const dsa_shape* shape, const dsa_mla_variant* variant, const uint16_t* q,
                                 const uint16_t* kv, const int32_t* topk_idx, const uint16_t* W_UV,
                                 const uint16_t* gate, const uint16_t* out, const float* lse,
                                 const uint16_t* dout, float* dq, float* dkv, float* dW_UV, float* dgate,
                                 float* dsink, void* workspace, size_t workspace_bytes, void* stream);

/* dsa_sparse_mla_bwd_ex given the forward's latent attention output o_lat [rows, H, 512] bf16
 * (16-byte aligned), as dsa_sparse_attention_latent(_ex) wrote it for the same q, kv, topk_idx and
 * variant. dW_UV = sum over rows of o_lat^T (sigmoid(gate) * dout) then reads these rows instead of
 * recomputing the attention for them; with the forward's own o_lat every output is the one
 * dsa_sparse_mla_bwd_ex gives (the attention is deterministic). This trades rows * H * 1024 bytes
 * kept from the forward for one attention pass. o_lat must not be NULL (DSA_ERR_INVALID_ARG).
 * Other arguments, outputs and workspace as dsa_sparse_mla_bwd_ex. */
dsa_status dsa_sparse_mla_bwd_saved(const dsa_shape* shape, const dsa_mla_variant* variant, const uint16_t* q,
                                    const uint16_t* kv, const int32_t* topk_idx, const uint16_t* W_UV,
                                    const uint16_t* gate, const uint16_t* out, const float* lse,
                                    const uint16_t* o_lat, const uint16_t* dout, float* dq, float* dkv,
                                    float* dW_UV, float* dgate, float* dsink, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Static English text of a status. Never NULL. */
const char* dsa_status_string(dsa_status status);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
