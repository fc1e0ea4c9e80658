// Launch wrappers of the gfx950 kernels (internal to libdsa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kIdxMaxSeg = 64;  // row segments per indexer launch
constexpr int kIdxKeyPad = 128; // LNk rows past T in the workspace: the indexer stages whole 128-key
                                // chunks (the last one reaching up to 127 rows past the last key)
                                // and never scores those rows
constexpr int kIdxMaxTopk = 2048;  // largest k the indexer's buffers are sized for
constexpr int kIdxSlots = 256;  // candidate-list slots: one per indexer workgroup resident at a time
                                // (one per CU on MI355X); launches check residency against this
constexpr int kIdxCap = 4608;   // candidate-list capacity of one indexer row
constexpr int kIdxSlotWords = 8 * 2 * (kIdxCap + 64);  // int32 words of one slot: 8 rows' candidate score
                                                      // keys and token indices (capacity + 64 of each)

struct IndexArgs {
  const uint16_t* q_I;   // [nrows, H_I, d_I] local rows
  const uint16_t* w;     // [nrows, H_I]
  const uint16_t* LNk;   // [T + kIdxKeyPad, d_I]; rows past T are staged but never scored
  int32_t* topk_idx;     // [nrows, k]
  const int32_t* cu;     // device cu_seqlens or nullptr
  int n_docs;
  int T;
  int row0;              // global token of local row 0
  int nrows;
  int k;
  const uint8_t* q8;     // FP8 indexer: [nrows, H_I, d_I] E4M3 codes of q_I
  const float* sq;       //   [nrows, H_I] their power-of-two scales
  const uint8_t* LNk8;   //   [T + kIdxKeyPad, d_I] E4M3 codes of LNk
  const float* sk;       //   [T + kIdxKeyPad] their power-of-two scales
  int32_t* cand;         // candidate lists (score keys, token indices): n_slots slots of kIdxSlotWords words each
  int* slot_flags;       // [n_slots] 1 while a workgroup holds the slot; zeroed by the prologue
  int n_slots;
  // Rows that need a selection, as segments of consecutive local rows of one document each.
  // Segment s: rows [seg_r0, seg_r0 + seg_m), document start token seg_b, blocks
  // [seg_blk0[s], seg_blk0[s + 1]). paired != 0: each block takes 4 of the longest and 4 of the
  // shortest rows left in its segment; else 8 consecutive rows, longest first.
  int nseg;
  int paired;
  int seg_r0[kIdxMaxSeg];
  int seg_m[kIdxMaxSeg];
  int seg_b[kIdxMaxSeg];
  int seg_blk0[kIdxMaxSeg + 1];
  const uint16_t* k_raw; // key LayerNorm fused into the key-chunk loads: [T, d_I] the raw k_I,
  const float* ln_gamma; //   its optional affine weight and bias [d_I] (nullptr: none)
  const float* ln_beta;
  double ln_eps;
};

struct MlaArgs {
  const uint16_t* q;     // [nrows, H, 576] local rows
  const uint16_t* kv;    // [T, 576]
  const int32_t* idx;    // [nrows, k]
  uint16_t* o_lat;       // [chunk_rows, H, 512] workspace, local to the chunk
  float* lse;            // [nrows, H] or nullptr
  const float* sink;     // [H] per-head sink logits (natural-log units) or nullptr: no sink
  const int32_t* cu;
  int n_docs;
  int T;
  int row0;              // global token of local row 0
  int chunk_r0;          // first local row of this chunk
  int chunk_rows;
  int k;
  int H;
  float scale_log2;      // softmax scale * log2(e)
};

struct UpArgs {
  const uint16_t* o_lat;  // [chunk_rows, H, 512]
  const uint16_t* W_UV;   // [H, 512, 128]
  const uint16_t* gate;   // [nrows, H], or [nrows, H, 128] when gate_per_dim
  uint16_t* out;          // [nrows, H, 128]
  int chunk_r0;
  int chunk_rows;
  int H;
  int gate_per_dim;       // 0: one gate logit per (row, head); 1: one per output element
};

struct AbsorbArgs {
  const uint16_t* q_nope;  // [rows, H, 128]
  const uint16_t* q_pe;    // [rows, H, 64], or nullptr: no pass-through dims
  const uint16_t* W_UK;    // [H, 512, 128]
  uint16_t* q;             // [rows, H, out_stride]
  int rows;
  int H;
  int out_stride;          // 576 (the latent query), or 512 (no pass-through dims)
};

struct GemmArgs {
  const uint16_t* A;  // [M, K] bf16, K contiguous
  const uint16_t* B;  // [N, K] bf16, K contiguous
  uint16_t* C;        // [M, N] bf16
  int M, N, K;        // N a multiple of 256, K a multiple of 64
};

struct BwdPrepArgs {
  const uint16_t* dout;  // [nrows, H, 128] bf16, caller rows
  const uint16_t* out;   // [nrows, H, 128] bf16, the forward's output
  const uint16_t* gate;  // [nrows, H] bf16, or [nrows, H, 128] with gate_per_dim
  uint16_t* d_o;         // [rows, H, 128] bf16, chunk-local: sigma(g) dout
  float* delta;          // [rows, H], chunk-local: sum_d dout * out
  float* dgate;          // [nrows, H] (or [nrows, H, 128]), caller rows
  int rows;              // rows of this chunk
  int H;
  int row_off;           // first caller row of the chunk
  int gate_per_dim;
  const float* sink;     // [H] or nullptr
  const float* lse;      // [nrows, H], caller rows (read with a sink)
  float* sterm;          // [rows, H], chunk-local, with a sink: -exp(sink - lse) * delta
};

// dsink[h] += sum over the chunk's rows of sterm[row, h]: one workgroup per head.
struct SinkSumArgs {
  const float* sterm;    // [rows, H]
  float* dsink;          // [H], added to
  int rows;
  int H;
};

struct BwdArgs {
  const uint16_t* q;       // [nrows, H, 576]
  const uint16_t* kv;      // [T, 576]
  const int32_t* idx;      // [nrows, k]
  const float* lse;        // [nrows, H] natural log, from the forward
  const float* delta;      // [chunk_rows, H]
  const uint16_t* do_lat;  // [chunk_rows, H, 512]
  float* dq;               // [nrows, H, 576]
  uint16_t* g;             // [chunk_rows, g_stride, 2H] bf16 per selected key: dS' of the H heads, then P
  int g_stride;            // keys per row of g: k rounded up to 32
  const int32_t* cu;
  int n_docs;
  int T;
  int row0;                // global token of local row 0
  int chunk_r0;
  int chunk_rows;
  int k;
  int H;                   // 96
  float scale;
};

// The dkv contribution of each (row r, selected key j) of a row chunk, over all H heads, from g:
//   contrib(r, j) = dS'[r, j, :] q[r] + P[r, j, :] do_lat[r]  (576 floats)
// stored, for the pairs with a usable index, at the pair's position in key order (from the pair sort),
// so that k_dkv_sum reads each key's contributions contiguously.
struct DkvArgs {
  const uint16_t* g;       // as BwdArgs::g
  const uint16_t* q;       // [nrows, H, 576]
  const uint16_t* do_lat;  // [chunk_rows, H, 512]
  const int32_t* pos;      // [chunk_rows * k] position of pair r * k + j in key order, or -1 (DkvListArgs::list)
  uint16_t* contrib;       // [3][chunk_rows * k][192] bf16: group q holds dims 192q .. 192q + 191 of the pair at position p
  const int32_t* cu;
  int n_docs;
  int T;
  int row0;
  int chunk_r0;
  int chunk_rows;
  int k;
  int g_stride;
};

// Per-key lists of a row chunk's (row, j) pairs (a counting sort by key index), and their sum into dkv.
constexpr int kPairScanTile = 4096;  // keys per workgroup of the scan over count
struct DkvListArgs {
  const int32_t* idx;      // [nrows, k]
  const int32_t* cu;
  int n_docs;
  int T;
  int row0;
  int chunk_r0;
  int chunk_rows;
  int k;
  int* count;              // [T] pairs per key (zeroed before the count pass)
  int* start;              // [T + 1] exclusive prefix sums of count
  int* bsum;               // [ceil(T / kPairScanTile)] count sums of the scan's blocks
  int* list;               // [chunk_rows * k] position of pair r * k + j in key order (-1: no usable key);
                           // the count pass leaves the pair's rank among its key's pairs there first
  const uint16_t* contrib; // as DkvArgs::contrib
  float* dkv;              // [T, 576], added to
};

struct DwArgs {
  const uint16_t* o_lat;  // [rows, H, 512] chunk-local
  const uint16_t* d_o;    // [rows, H, 128] chunk-local
  float* dW;              // [H, 512, 128], added to
  int rows;
  int H;
};

// Key LayerNorm of all T keys into LNk, and the outputs of the rows with at most k causal keys.
// do_ln = false leaves the key LayerNorm out (the fused-LN indexer normalises keys as it stages them).
hipError_t launch_index_prologue(const uint16_t* k_I, const float* gamma, const float* beta, double eps, int d_I,
                                 uint16_t* LNk, const IndexArgs& a, hipStream_t st, bool do_ln = true);
hipError_t launch_index_topk(const IndexArgs& a, int H_I, int d_I, bool fp8, hipStream_t st, bool fused_ln = false);
// FP8 indexer operands: n rows of 128 bf16 values -> E4M3 codes and the rows' power-of-two scales
// (smallest 2^e with amax * 2^-e <= 448). Two independent row sets in one launch (n2 may be 0).
hipError_t launch_quantize_fp8(const uint16_t* x1, int64_t n1, uint8_t* q1, float* s1, const uint16_t* x2, int64_t n2,
                               uint8_t* q2, float* s2, hipStream_t st);
int index_blocks(int m, int paired);  // blocks of a segment of m rows
hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t st);
hipError_t launch_up_gate(const UpArgs& a, hipStream_t st);
hipError_t launch_q_absorb(const AbsorbArgs& a, hipStream_t st);
hipError_t launch_gemm_nt(const GemmArgs& a, hipStream_t st);
hipError_t launch_bwd_prep(const BwdPrepArgs& a, hipStream_t st);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_sparse_mla_bwd(const BwdArgs& a, hipStream_t st);
hipError_t launch_dkv(const DkvArgs& a, hipStream_t st);
// count[key] = pairs of the chunk selecting key; start = exclusive scan;
// list = each pair's position in key order. Before k_dkv, which stores at those positions.
hipError_t launch_pairs_sort(const DkvListArgs& a, hipStream_t st);
// dkv[key] += the sum of the key's contributions (positions start[key] .. start[key + 1] - 1).
hipError_t launch_dkv_sum(const DkvListArgs& a, hipStream_t st);
hipError_t launch_sink_sum(const SinkSumArgs& a, hipStream_t st);
hipError_t launch_dwuv(const DwArgs& a, hipStream_t st);

}  // namespace dsa
