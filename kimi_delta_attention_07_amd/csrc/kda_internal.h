// Internal interface between the C ABI (kda_abi.cpp) and the HIP kernels.
// Parameter blocks are passed by value to the launchers; every pointer is a
// device pointer already validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Chunk geometry of the prefill path (fixed: head dim 128, 64-token chunks).
constexpr int kChunk = 64;
constexpr int kHeadDim = 128;
constexpr int kTileV = 16;                       // value columns per scan wave
constexpr int kTilesV = kHeadDim / kTileV;       // 8 scan waves per (sequence, head)

// Per-(chunk, head) record written by the prepare stage, read by the scan.
// All operands are stored as MFMA fragments (64 lanes x 16 B each) so both
// stages move them with whole-wave, fully coalesced 16-byte accesses.
//   W   16 fragments (tokens m 0..3 x channel k-step s 0..3): -W = -T beta (K e^G)
//   Qg  16 fragments (m x s):                                  Q e^G
//   Kg  16 fragments (channel tile 0..7 x token k-step 0..1):  (K e^{G_L - G})^T
//   P    8 fragments (m x token k-step 0..1):                  tril(Q e^G (K e^-G)^T)
//   U   32 fragments of 64 x 4 bf16 (value tile 0..7 x m):     T beta V
//   gL  128 fp32:                                               e^{G_L}
constexpr size_t kFragBytes = 64 * 16;
constexpr size_t kOffW = 0;
constexpr size_t kOffQg = kOffW + 16 * kFragBytes;
constexpr size_t kOffKg = kOffQg + 16 * kFragBytes;
constexpr size_t kOffP = kOffKg + 16 * kFragBytes;
constexpr size_t kOffU = kOffP + 8 * kFragBytes;
constexpr size_t kOffGL = kOffU + 32 * 64 * 8;
constexpr size_t kChunkRecordBytes = kOffGL + kHeadDim * 4;   // 74,240 B

struct ChunkInfo {
    int32_t start;  // first token (absolute, in the packed batch)
    int32_t len;    // 1..64
    int32_t seq;    // sequence index
    int32_t first;  // 1 for the first chunk of its sequence
};

struct PrologueParams {
    int T, H, d, K, act, n_seqs;
    float eps;
    const int32_t *cu;  // [n_seqs+1]
    const void *q_raw, *k_raw, *v_raw, *beta_logit, *gate_logit;
    const float *conv_w, *cache_in;
    float *cache_out;
    void *q_out, *k_out, *v_out, *gate_out;
    float *beta_out;
};

// Batches of up to kPlanSeqs sequences carry their chunk table in the kernel
// arguments (built on the host from cu_seqlens_host), so no table kernel runs.
constexpr int kPlanSeqs = 128;
static_assert(kPlanSeqs <= 256, "plan_order holds sequence numbers in 8 bits");

struct ChunkParams {
    int T, H, n_seqs, n_chunks;
    float scale;
    // fused prefill only: raw inputs of the short conv, read by the prepare
    // kernel, and raw gate logits (sigmoid applied by the scan)
    int K, act;
    float eps;
    const uint16_t *q_raw, *k_raw, *v_raw, *beta_logit;
    const float *conv_w, *cache_in;
    float *cache_out;           // written by each sequence's last chunk when set
    int gate_is_logit;
    const int32_t *cu;          // [n_seqs+1] device
    int32_t *chunk_off;         // [n_seqs+1] in workspace
    ChunkInfo *chunk_info;      // [n_chunks] in workspace
    unsigned char *records;     // [H][n_chunks][kChunkRecordBytes] in workspace
    const uint16_t *q, *k, *v, *log_alpha, *gate;   // bf16 bit patterns
    const float *beta;
    const float *s0;
    float *s_final;
    uint16_t *out;
    // small batches: first chunk of each sequence and cu_seqlens, [n_seqs+1],
    // and the scan's dispatch order, sequences by decreasing chunk count
    int plan_in_args;
    int32_t plan_off[kPlanSeqs + 1];
    int32_t plan_cu[kPlanSeqs + 1];
    uint8_t plan_order[kPlanSeqs];
};

struct DecodeParams {
    int batch, H, d, K, act, n_slots;
    float eps, scale;
    const int32_t *slot_idx;
    const void *q_raw, *k_raw, *v_raw, *log_alpha, *beta_logit, *gate_logit;
    const float *conv_w;
    float *conv_cache, *state;
    void *out;
};

// Backward of the chunk path.  Per (chunk, head) the workspace holds fp32
// row-major matrices (kBwdFloats floats; layout in backward.hip): the chunk's
// WY quantities, its entry state S0 and U from a forward state pass, the
// state gradient at its end, dO and dU from a backward state pass, and
// scratch for the per-chunk gradient products.
struct BwdParams {
    ChunkParams c;              // geometry, chunk table, forward inputs (q, k, v, log_alpha, beta, gate, s0)
    float *buf;                 // [n_chunks * H][kBwdFloats]
    const uint16_t *dy;         // [T][H][128] bf16: gradient of the output
    const float *ds_final;      // [n_seqs][H][128][128] or null: gradient of the final state
    float *dq, *dk, *dv, *dla;  // [T][H][128]
    float *dbeta;               // [T][H]
    float *dgate;               // [T][H][128], null when there is no gate
    float *ds0;                 // [n_seqs][H][128][128] or null
};
// Backward of the prologue (conv + activation, L2 norm, sigmoids).
struct PrologueBwdParams {
    int T, H, d, K, act, n_seqs;
    float eps;
    const int32_t *cu;                          // [n_seqs+1] device
    const void *q_raw, *k_raw, *v_raw;          // [T][H][d] in the forward's dtype
    const float *conv_w, *cache_in;             // [3][H*d][K]; NULL or [n_seqs][3][K-1][H*d]
    const void *beta_logit, *gate_logit;        // [T][H]; NULL or [T][H][d]
    const float *dq, *dk, *dv, *dbeta, *dgate;  // gradients reaching the prologue's outputs
    float *dq_raw, *dk_raw, *dv_raw;            // [T][H][d]
    float *dconv_w, *dcache_in;                 // [3][H*d][K]; NULL or as cache_in
    float *dbeta_logit, *dgate_logit;           // [T][H]; NULL or [T][H][d]
    void *workspace;                            // prologue_bwd_workspace_bytes()
    float *dpre, *dw_part;                      // carved from the workspace by the launcher
};
// Linear maps of the mixer: C = A B^T, A [M][K], B [N][K] bf16 (K contiguous,
// K % 8 == 0), fp32 accumulation, bf16 out.  epi 0: out [M][N]; epi 1: the KDA
// input projection, columns split into q, k, v, gate, decay (H d each) and
// beta (H) segments written to seg[0..5] ([M][width] each), the decay segment
// through log alpha = -exp(a_log[h]) softplus(z + bias[h d + c]).
struct ProjParams {
    int M, N, K;
    const uint16_t *a, *b;
    int epi;
    uint16_t *out;
    int H, d;
    uint16_t *seg[6];
    const float *a_log, *bias;   // [H], [H d]; either may be null
};
hipError_t launch_gemm(const ProjParams &p, hipStream_t s);

// MLA decode token (mla.hip): bf16 q, k_new, v_new, gate, caches and output
struct MlaParams {
    int batch, H, H_kv, dqk, dv, max_len, n_split;
    float scale;
    const int32_t *cache_len;                 // [batch], device
    const void *q, *k_new, *v_new, *gate;     // gate may be null
    void *k_cache, *v_cache, *out;
    float *ws_ml;                             // [batch][H][n_split][2]: max, sum
    float *ws_acc;                            // [batch][H][n_split][dv]
};
int mla_split_tokens();
hipError_t launch_mla_decode(const MlaParams &p, bool vec, hipStream_t s);

size_t prologue_bwd_workspace_bytes(int H, int d, long T);
hipError_t launch_prologue_backward(PrologueBwdParams p, int dtype, hipStream_t s);

hipError_t launch_chunk_plan(const ChunkParams &p, hipStream_t s);
hipError_t launch_chunk_backward(const BwdParams &p, hipStream_t s);
size_t bwd_workspace_bytes(int H, int n_seqs, long n_chunks);
void bwd_workspace_carve(void *ws, int H, int n_seqs, long n_chunks, BwdParams &p);

// dtype codes match kda_dtype: 0 = fp32, 1 = bf16.
hipError_t launch_prologue(const PrologueParams &p, int dtype, hipStream_t s);
hipError_t launch_chunk_prepare(const ChunkParams &p, hipStream_t s);
hipError_t launch_prefill_prepare(const ChunkParams &p, hipStream_t s);   // fused conv/L2/gates
hipError_t launch_conv_cache_out(const PrologueParams &p, int dtype, hipStream_t s);
hipError_t launch_chunk_scan(const ChunkParams &p, hipStream_t s);
hipError_t launch_decode(const DecodeParams &p, int in_dtype, int out_dtype, hipStream_t s);

// Workspace carving shared by the two chunk stages.
size_t chunk_workspace_bytes(int H, int n_seqs, long n_chunks);
void chunk_workspace_carve(void *ws, int H, int n_seqs, long n_chunks, ChunkParams &p);

}  // namespace kda
