// Launch interface of the libdllm HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dllm {

enum DType { F32 = 0, BF16 = 1 };

// ---------------------------------------------------------------- GEMM epilogues
// Every GEMM computes acc[m][vc] = sum_k X[m][k] * W[row(vc)][k] over "virtual" output
// columns vc in tiles of 128, then hands a whole fp32 tile to one of these epilogues.
enum EpiKind {
  EPI_STORE = 0,   // y T [M][ldy]      = acc
  EPI_F32 = 1,     // y fp32 [M][ldy]   = scale * acc
  EPI_RESID = 2,   // y fp32 [M][ldy]  += acc                (residual add)
  EPI_SWIGLU = 3,  // virtual tile t = 64 gate rows + 64 up rows; y T [M][F] = silu(g) * u
  EPI_QKV = 4      // RoPE on q/k, scatter q to [B][Hq][R][D], k/v into the cache
};

struct EpiArgs {
  void* y = nullptr;
  int ldy = 0;
  float scale = 1.f;
  int F = 0;                       // SWIGLU: d_ffn
  // QKV
  void* qo = nullptr;              // T [B][Hq][R][D]
  void* kc = nullptr;              // T [B][Hkv][Sp][D]  (this layer's K)
  void* vtc = nullptr;             // T [B][Hkv][Sp/32][D][32]  (this layer's V, see vt_off)
  const float* rcos = nullptr;     // [S][D/2]
  const float* rsin = nullptr;
  int Hq = 0, Hkv = 0, D = 0, R = 0, pos0 = 0, Sp = 0;
  // Deferred RMS factor (skinny split-K reduction only): when rss is set, the GEMM input
  // was bf16(x * g) and row m of the result is multiplied by
  // 1 / sqrt(sum(rss[m][0..rseg)) / rd + reps) before the epilogue.
  const float* rss = nullptr;
  int rseg = 0, rd = 0;
  float reps = 0.f;
};

// The value cache holds V transposed and blocked by 32 keys: per (sequence, KV head),
// [Sp/32][D][32], so value (dim d, key k) sits at vt_off(d, k, D) and the 32 keys x D
// dims of one block are contiguous (Sp is a multiple of 32).
__host__ __device__ inline int64_t vt_off(int d, int k, int D) {
  return ((int64_t)(k >> 5) * D + d) * 32 + (k & 31);
}

enum GemmKind { GEMM_F32 = 0, GEMM_SKINNY = 1, GEMM_TILED = 2, GEMM_BIG = 3, GEMM_MID = 4 };
constexpr int kSkinnyRows = 64;  // bf16 GEMMs with at most this many rows stream weights
constexpr int kMidRows = 256;    // above kSkinnyRows and up to this many: one 256-row tile
constexpr int kBigTile = 256;    // output tile edge of the large-tile GEMM

// Where split-K partial sums live.  Plain: [split][M][N].  Blocked (skinny GEMM): per split,
// per 16-column group, one block of mrows x 16 floats in which row m, column c sits at
// ((mt*4 + r)*4 + g)*16 + c with m = 16 mt + 4 g + r, so that every store instruction of
// the producing wave writes 256 contiguous bytes.  Four consecutive columns starting at a
// multiple of 4 are contiguous in both layouts.  Partial column c is the GEMM's virtual
// output column vbase + c (vbase > 0 when only the trailing tiles were split).
struct PartView {
  const float* p = nullptr;
  int splits = 0;
  int blocked = 0;
  int mrows = 0;        // blocked: rows per block (16, 32 or 64)
  int M = 0, N = 0;     // plain: row stride is N
  int vbase = 0;        // a multiple of 128
  // virtual column order of the producing GEMM: 0 = 64-column groups (weight-streaming and
  // mid-size GEMMs: SwiGLU 32 gate + 32 up, QKV head dims 0-31, 64-95, 32-63, 96-127);
  // 1 = 128-column groups (large tiles: SwiGLU 64 gate + 64 up, QKV dims in order)
  int order = 0;
  __host__ __device__ int64_t split_stride() const {
    return blocked ? (int64_t)((N + 15) / 16) * mrows * 16 : (int64_t)M * N;
  }
  __host__ __device__ int64_t off(int m, int c) const {
    if (!blocked) return (int64_t)m * N + c;
    const int mt = m >> 4, g = (m & 15) >> 2, r = m & 3;
    return (int64_t)(c >> 4) * mrows * 16 + ((mt * 4 + r) * 4 + g) * 16 + (c & 15);
  }
};

#ifdef __HIPCC__
// Split-K sums for the reductions (reduce_epilogue, the fused LM-head confidence pass).
// Sum of split partials at (m, c..c+3), in split order.
__device__ __forceinline__ float4 sum_split4(const PartView& pv, int m, int c) {
  const int64_t stride = pv.split_stride();
  const float* p = pv.p + pv.off(m, c);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < pv.splits; s0 += 4) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = (s0 + u < pv.splits) ? *reinterpret_cast<const float4*>(p + (s0 + u) * stride)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + u < pv.splits) { s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w; }
  }
  return s;
}

// Deferred RMS factor of row m (1 when the input was already normalised); the segment
// sums are added in segment order.
__device__ __forceinline__ float row_rms_factor(const EpiArgs& e, int m) {
  if (e.rss == nullptr) return 1.f;
  const float* s = e.rss + (int64_t)m * e.rseg;
  float t = 0.f;
  for (int i = 0; i < e.rseg; ++i) t += s[i];
  return 1.0f / sqrtf(t / (float)e.rd + e.reps);
}
__device__ __forceinline__ float4 scale4(float4 v, float r) {
  return make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
}
#endif

struct GemmPlan {
  int kind = 0;
  int mt = 1;            // skinny: 16-row MFMA tiles per workgroup (1, 2 or 4)
  int ntn = 0, ntm = 0;  // tiles along N (virtual) and M
  int splits = 1, kchunk = 0;
  size_t part_floats = 0;  // split-K partial buffer
  int counters = 0;        // split-K arrival counters
  bool deferred = false;   // residual partials left for the next RMSNorm to add
  bool reduce = false;     // a reduce_epilogue launch finishes the split columns
  int ndp = 0;             // mid: leading tiles computed whole (direct epilogue); large
                           // tiles: leading column tiles computed whole, the rest split
  int units = 0;           // mid: work units (whole tiles, then tile x K-split pieces)
  bool tail_tiled = false; // large tiles: columns from ndp on run as 128x128 tiles
  PartView view(const float* part, int M, int N) const {
    PartView v;
    v.p = part; v.splits = splits; v.M = M;
    v.blocked = (kind == GEMM_SKINNY);
    v.mrows = mt * 16;
    v.vbase = (kind == GEMM_MID) ? ndp * 128 : (kind == GEMM_BIG ? ndp * kBigTile : 0);
    v.order = (kind == GEMM_BIG) ? 1 : 0;
    v.N = N - v.vbase;
    return v;
  }
};

GemmPlan gemm_plan(int dtype, int M, int Nv, int K, int epi);
// launch_gemm = launch_gemm_only + launch_reduce_epilogue when the plan asks for it
hipError_t launch_gemm(int dtype, int epi, const GemmPlan& p, const void* X, int ldx,
                       const void* W, int M, int Nv, int K, const EpiArgs& e, float* part,
                       int* counters, hipStream_t st);
hipError_t launch_gemm_only(int dtype, int epi, const GemmPlan& p, const void* X, int ldx,
                            const void* W, int M, int Nv, int K, const EpiArgs& e, float* part,
                            int* counters, hipStream_t st);
hipError_t launch_reduce_epilogue(int epi, const PartView& pv, const EpiArgs& e, hipStream_t st);

// ---------------------------------------------------------------- attention
struct AttnPlan {
  int kind = 0;          // 0: fp32 simple, 1: bf16 split-KV (R <= 64), 2: bf16 flash,
                         // 3: bf16 grouped-query split-KV (R <= 32, 2 <= Hq/Hkv <= 8)
  int nqt = 0, nchunk = 0, nsub = 0;
  int ck = 0;            // grouped-query: keys per chunk
  int nw = 4;            // split-KV: waves per workgroup (4 or 8)
  size_t part_floats = 0;
  int counters = 0;      // unused: chunk partials are merged by a second kernel
};
AttnPlan attn_plan(int dtype, int B, int Hq, int Hkv, int R, int S, int D);
// Partial floats of the attention plan for the largest need over every Hkv dividing Hq
// (the grouped-query plan may use more, shorter chunks than the plan for Hkv = Hq).
size_t attn_part_floats_any_hkv(int dtype, int B, int Hq, int R, int S, int D);
hipError_t launch_attention(int dtype, const AttnPlan& p, const void* q, const void* k,
                            const void* vt, void* o, int B, int Hq, int Hkv, int R, int S,
                            int Sp, int D, float* part, int* counters, hipStream_t st);

// ---------------------------------------------------------------- confidence / unmask
struct ConfPlan {
  int it = 1;  // 8-element loads per thread per pass (1, 2, 4 or 8)
  int nsplit = 1, chunk = 0;
  size_t part_elems = 0;  // per array (m, s, idx)
};
ConfPlan conf_plan(int rows, int V, int B);
hipError_t launch_conf_unmask(int ldtype, const ConfPlan& p, const void* logits, int B, int K,
                              int V, int mask_id, float tau, int* tokens, int ld_tokens,
                              float* conf, int* argmax, int* n_unmasked, int* remaining,
                              int* unmasked_idx, float* pm, float* ps, int* pi, hipStream_t st);
// The same with pass 1 fused into the LM head's split-K reduction (partials pv, epilogue
// args e as for reduce_epilogue<EPI_F32>); logits (row stride e.ldy) are written only if
// non-null.  Usable when lm_conf_fusable(p, V).
bool lm_conf_fusable(const ConfPlan& p, int V);
hipError_t launch_lm_conf_unmask(const ConfPlan& p, const PartView& pv, const EpiArgs& e,
                                 float* logits, int B, int K, int V, int mask_id, float tau,
                                 int* tokens, int ld_tokens, float* conf, int* argmax,
                                 int* n_unmasked, int* remaining, int* unmasked_idx, float* pm,
                                 float* ps, int* pi, hipStream_t st);

// ---------------------------------------------------------------- small kernels
hipError_t launch_rope_table(float* cosb, float* sinb, int S, int D, float theta, hipStream_t st);
// x[j] = embed[tokens[b*S + r0 + i]] (fp32), h[j] = rmsnorm(x[j]) * g  for j = b*R + i
hipError_t launch_embed_norm(int dtype, const int* tokens, int S, int r0, int R, int B,
                             const void* embed, const void* g, float eps, int d, int V, float* x,
                             void* h, hipStream_t st);
// h[j] = rmsnorm(x[in_row(j)]) * g, in_row(j) = (j / Kout) * Rin + j % Kout, j < rows.
// With pv.splits > 0, first x[in_row] += the pending split partials of that row (split
// order), written back into x.
hipError_t launch_rmsnorm(int dtype, float* x, int rows, int Rin, int Kout, const void* g,
                          float eps, int d, void* h, const PartView& pv, hipStream_t st);
// RMSNorm with the row factor deferred to the consumer: for j < rows, x[in_row(j)] += the
// pending split partials (split order), h[j] = x[in_row(j)] * g (no 1/rms), and
// rss[j][s] = the sum of squares of columns [s*kFoldSeg, (s+1)*kFoldSeg) of that row.
// grid (ceil(d / kFoldSeg), rows): every CU takes a share of the rows.
constexpr int kFoldSeg = 512;
hipError_t launch_fold_scale(int dtype, float* x, int rows, int Rin, int Kout, const void* g,
                             int d, void* h, float* rss, const PartView& pv, hipStream_t st);
// y[m][c] += sum over splits of the partials at (m, c), in split order (y is [M][N] fp32)
hipError_t launch_fold_partials(float* y, const PartView& pv, hipStream_t st);
hipError_t launch_fill_i32(int* p, int64_t n, int v, hipStream_t st);
// Cosine similarity of cached and fresh K/V per layer (positions outside [x0, x1)):
// out [L][2][2] = {K mean, K min}, {V mean, V min}; part: L * 2 * B * Hkv * 3 doubles.
hipError_t launch_staleness(int dtype, const void* cached, const void* fresh, int L, int B,
                            int Hkv, int S, int Sp, int D, int x0, int x1, double* part,
                            float* out, hipStream_t st);
hipError_t launch_synth_fill(void* dst, int64_t n, int dtype, uint64_t seed, uint32_t tid,
                             double stdv, int mode, hipStream_t st);

}  // namespace dllm
