// Vocab-wide confidence (max softmax probability) and argmax per block row, fused with
// the threshold-unmask compaction of each sequence's block.
//
// Confidence is the probability the model gives its most likely token; every masked
// position of the block at or above the threshold is decoded this step, the others wait
// (ccyt168.com Fast-dLLM article, section 1.2 "Confidence-Aware Parallel Decoding";
// techwalker.com explainer, "Solving the quality loss of parallel decoding").
//
// Two passes.  Pass 1, grid (nsplit, rows): each workgroup streams one slice of one row
// with 16-byte loads (all of a thread's loads in flight together), takes the slice's
// maximum, then the sum of exp(z - max), and writes a per-(row, slice) (max, sum,
// argmax) triple.  Pass 2, one workgroup per sequence, merges each row's slice triples
// (a few lanes per row, then a lane butterfly) and runs the unmask rule with wave
// ballots.  Cross-lane steps use DPP lane permutes and fixed combination orders; there
// are no atomics, so results are bit-identical from run to run.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dllm {

struct Trip {
  float m;    // max logit (mask id excluded), -inf if none seen
  float s;    // sum of exp(z - m)
  int idx;    // lowest id reaching m
};

__device__ __forceinline__ Trip merge(Trip a, Trip b) {
  if (b.m == -INFINITY) return a;
  if (a.m == -INFINITY) return b;
  Trip r;
  r.m = fmaxf(a.m, b.m);
  r.s = a.s * __builtin_amdgcn_exp2f((a.m - r.m) * kLog2e) +
        b.s * __builtin_amdgcn_exp2f((b.m - r.m) * kLog2e);
  r.idx = (a.m > b.m) ? a.idx : (b.m > a.m) ? b.idx : min(a.idx, b.idx);
  return r;
}

// Fold a group of n consecutive values (ids id0..id0+n-1, increasing) into t.
__device__ __forceinline__ void fold(Trip& t, const float* v, int n, int id0, int mask_id) {
  float lm = -INFINITY;
  int li = 0x7fffffff;
  float vv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < n) {
      float x = (id0 + e == mask_id) ? -INFINITY : v[e];
      vv[e] = x;
      if (x > lm) { lm = x; li = id0 + e; }
    } else {
      vv[e] = -INFINITY;
    }
  }
  if (lm == -INFINITY) return;
  if (lm > t.m) {
    t.s = (t.m == -INFINITY) ? 0.f : t.s * __builtin_amdgcn_exp2f((t.m - lm) * kLog2e);
    t.m = lm;
    t.idx = li;
  }
  float ml = t.m * kLog2e;
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc += __builtin_amdgcn_exp2f(fmaf(vv[e], kLog2e, -ml));
  t.s += acc;
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  u32x4 a = *reinterpret_cast<const u32x4*>(p);
  uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}

constexpr int kConfThreads = 256;
constexpr int kConfMaxParts = 2048;  // K * nsplit per sequence (finalize stages them in LDS)
constexpr int kConfMaxSplit = 64;

// Workgroup merge of per-thread (max m, sum s of exp(z - m)) pairs: the slice maximum M,
// the sum rescaled to M, and the lowest id reaching M, which only threads with m == M
// look for (find_idx returns a thread's lowest such id).  All threads must call it.
template <typename F>
__device__ __forceinline__ Trip block_merge(float m, float s, F find_idx, float* rm, float* rs,
                                            int* ri) {
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  constexpr int NW = kConfThreads / kWave;
  const float wm = wave_max_dpp(m);
  if (lane == 0) rm[w] = wm;
  __syncthreads();
  float M = rm[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, rm[i]);
  if (M == -INFINITY) return Trip{-INFINITY, 0.f, 0x7fffffff};  // uniform: empty slice
  const float sr = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - M) * kLog2e);
  const int idx = (m == M) ? find_idx(M) : 0x7fffffff;
  const float ws = wave_sum_dpp(sr);
  const int wi = wave_min_dpp(idx);
  if (lane == 0) { rs[w] = ws; ri[w] = wi; }
  __syncthreads();
  Trip r{M, rs[0], ri[0]};
#pragma unroll
  for (int i = 1; i < NW; ++i) { r.s += rs[i]; r.idx = min(r.idx, ri[i]); }
  return r;
}

// The slice triple from values held in registers: thread tid holds ids
// lo + (j * kConfThreads + tid) * 8 + e (j < IT, e < 8) in v[j][e]; ids past hi and the
// mask id are dropped.  The thread's maximum first, then one exp per value against it,
// and the argmax search only in threads that hold the slice maximum.
template <int IT>
__device__ __forceinline__ Trip slice_trip(float (&v)[IT][8], int lo, int hi, int mask_id,
                                           float* rm, float* rs, int* ri) {
  constexpr int SPAN = IT * kConfThreads * 8;
  const int tid = threadIdx.x;
  if (hi - lo < SPAN || (lo <= mask_id && mask_id < hi)) {  // uniform: ragged or mask slice
#pragma unroll
    for (int j = 0; j < IT; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = lo + (j * kConfThreads + tid) * 8 + e;
        if (i >= hi || i == mask_id) v[j][e] = -INFINITY;
      }
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < IT; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, v[j][e]);
  float s = 0.f;
  if (m != -INFINITY) {
    const float ml = m * kLog2e;
#pragma unroll
    for (int j = 0; j < IT; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += __builtin_amdgcn_exp2f(fmaf(v[j][e], kLog2e, -ml));
  }
  auto find = [&](float M) {
    int best = 0x7fffffff;
#pragma unroll
    for (int j = IT - 1; j >= 0; --j)
#pragma unroll
      for (int e = 7; e >= 0; --e)
        if (v[j][e] == M) best = lo + (j * kConfThreads + tid) * 8 + e;
    return best;
  };
  return block_merge(m, s, find, rm, rs, ri);
}

// Pass 1, one workgroup per (slice, row).  A slice is chunk consecutive ids (the last one
// shorter).  When chunk == IT * 2048 (the usual plan) each thread holds its IT groups of 8
// values in registers: maximum first, then one exp per value, and the argmax search only
// in threads that hold the slice maximum.  Longer slices (very large vocabularies) fold
// online, one group of 8 at a time.  The mask id never counts.
template <typename T, int IT>
__global__ __launch_bounds__(kConfThreads) void conf_partials_kernel(
    const T* __restrict__ logits, int V, int mask_id, int nsplit, int chunk, float* pm,
    float* ps, int* pi) {
  __shared__ float rm[kConfThreads / kWave], rs[kConfThreads / kWave];
  __shared__ int ri[kConfThreads / kWave];
  const int split = blockIdx.x, row = blockIdx.y;
  const int lo = split * chunk;
  const int hi = min(V, lo + chunk);
  const T* zr = logits + (int64_t)row * V;
  const int tid = threadIdx.x;
  constexpr int SPAN = IT * kConfThreads * 8;

  Trip t;
  if ((V % 8) == 0 && chunk == SPAN) {
    float v[IT][8];
#pragma unroll
    for (int j = 0; j < IT; ++j)  // clamped in-row address; values past hi are dropped
      load8<T>(zr + min(lo + (j * kConfThreads + tid) * 8, V - 8), v[j]);
    t = slice_trip<IT>(v, lo, hi, mask_id, rm, rs, ri);
  } else {
    Trip u{-INFINITY, 0.f, 0x7fffffff};
    if ((V % 8) == 0) {
      for (int base = lo; base < hi; base += SPAN) {
        float v[IT][8];
#pragma unroll
        for (int j = 0; j < IT; ++j)
          load8<T>(zr + min(base + (j * kConfThreads + tid) * 8, V - 8), v[j]);
#pragma unroll
        for (int j = 0; j < IT; ++j) {
          const int i = base + (j * kConfThreads + tid) * 8;
          fold(u, v[j], min(max(hi - i, 0), 8), i, mask_id);
        }
      }
    } else {
      for (int i = lo + tid; i < hi; i += kConfThreads) {
        float v[8];
        v[0] = Elt<T>::load(zr, i);
        fold(u, v, 1, i, mask_id);
      }
    }
    t = block_merge(u.m, u.s, [&](float) { return u.idx; }, rm, rs, ri);
  }
  if (tid == 0) {
    const int64_t o = (int64_t)row * nsplit + split;
    pm[o] = t.m;
    ps[o] = t.s;
    pi[o] = t.idx;
  }
}

// Pass 1 fused with the LM head's split-K reduction: the logits of the slice are formed
// in registers from the weight-streaming GEMM's partials, exactly as reduce_epilogue
// forms them (the splits summed in order, times the row's deferred RMS factor, times the
// logit scale), stored only when the caller wants them, and reduced to the slice triple.
// This removes the fp32 logits round trip through memory.  Needs V % 8 == 0 and
// chunk == IT * kConfThreads * 8 (the plan's usual shape).
template <int IT>
__global__ __launch_bounds__(kConfThreads) void lm_conf_partials_kernel(
    PartView pv, EpiArgs e, float* __restrict__ logits, int V, int mask_id, int nsplit,
    int chunk, float* pm, float* ps, int* pi) {
  __shared__ float rm[kConfThreads / kWave], rs[kConfThreads / kWave];
  __shared__ int ri[kConfThreads / kWave];
  const int split = blockIdx.x, row = blockIdx.y;
  const int lo = split * chunk;
  const int hi = min(V, lo + chunk);
  const int tid = threadIdx.x;
  const float r = row_rms_factor(e, row);
  float v[IT][8];
#pragma unroll
  for (int j = 0; j < IT; ++j) {
    const int c = min(lo + (j * kConfThreads + tid) * 8, V - 8);  // clamped; dropped past hi
    const float4 a = scale4(sum_split4(pv, row, c), r);
    const float4 b = scale4(sum_split4(pv, row, c + 4), r);
    v[j][0] = a.x * e.scale; v[j][1] = a.y * e.scale; v[j][2] = a.z * e.scale; v[j][3] = a.w * e.scale;
    v[j][4] = b.x * e.scale; v[j][5] = b.y * e.scale; v[j][6] = b.z * e.scale; v[j][7] = b.w * e.scale;
  }
  if (logits) {
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      const int c = lo + (j * kConfThreads + tid) * 8;
      if (c < hi) {  // hi and c are multiples of 8: all 8 in range
        float* o = logits + (int64_t)row * e.ldy + c;
        *reinterpret_cast<float4*>(o) = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(v[j][4], v[j][5], v[j][6], v[j][7]);
      }
    }
  }
  const Trip t = slice_trip<IT>(v, lo, hi, mask_id, rm, rs, ri);
  if (tid == 0) {
    const int64_t o = (int64_t)row * nsplit + split;
    pm[o] = t.m;
    ps[o] = t.s;
    pi[o] = t.idx;
  }
}

// Pass 2, one workgroup per sequence: stage its K * nsplit partials in LDS (all loads
// issued together, the block's tokens read first), merge each row's slices with G lanes
// per row (G = 8 for K <= 32, else 4; slices sp = g, g + G, ... per lane, then a lane
// butterfly), and apply the threshold rule with wave ballots (lane i = block position i).
template <int G>
__device__ __forceinline__ Trip merge_lanes(Trip a) {
  auto step = [&](auto perm) {
    Trip o{perm(a.m), perm(a.s), 0};
    o.idx = __float_as_int(perm(__int_as_float(a.idx)));
    a = merge(a, o);
  };
  step([](float x) { return dpp<0xB1>(x); });
  if constexpr (G >= 4) step([](float x) { return dpp<0x4E>(x); });
  if constexpr (G >= 8) step([](float x) { return dpp<0x141>(x); });
  return a;
}

__global__ __launch_bounds__(kConfThreads) void conf_finalize_kernel(
    int K, int nsplit, int mask_id, float tau, const float* pm, const float* ps, const int* pi,
    int* tokens, int ld_tokens, float* conf, int* argmax, int* n_unmasked, int* remaining,
    int* unmasked_idx) {
  __shared__ float fm[kConfMaxParts], fs[kConfMaxParts];
  __shared__ int fi[kConfMaxParts];
  __shared__ float rowc[kWave];
  __shared__ int rowi[kWave];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int* tb = tokens + (int64_t)b * ld_tokens;
  const int tok = (tid < K) ? tb[tid] : 0;
  const int nparts = K * nsplit;
  const int64_t pbase = (int64_t)b * K * nsplit;
  for (int e0 = 0; e0 < nparts; e0 += kConfThreads * 8) {
    float lm[8], ls[8];
    int li[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = min(e0 + u * kConfThreads + tid, nparts - 1);
      lm[u] = pm[pbase + e];
      ls[u] = ps[pbase + e];
      li[u] = pi[pbase + e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kConfThreads + tid;
      if (e < nparts) { fm[e] = lm[u]; fs[e] = ls[u]; fi[e] = li[u]; }
    }
  }
  __syncthreads();
  {
    const int G = (K <= kConfThreads / 8) ? 8 : 4;
    const int row = tid / G, g = tid % G;
    Trip a{-INFINITY, 0.f, 0x7fffffff};
    if (row < K)
      for (int sp = g; sp < nsplit; sp += G) {
        const int e = row * nsplit + sp;
        a = merge(a, Trip{fm[e], fs[e], fi[e]});
      }
    a = (G == 8) ? merge_lanes<8>(a) : merge_lanes<4>(a);
    if (g == 0 && row < K) {
      const float c = 1.0f / a.s;
      rowc[row] = c;
      rowi[row] = a.idx;
      conf[b * K + row] = c;
      argmax[b * K + row] = a.idx;
    }
  }
  __syncthreads();
  if (tid >= kWave) return;

  const int i = tid;
  const bool active = i < K;
  const float c = active ? rowc[i] : 0.f;
  const int am = active ? rowi[i] : 0;
  const bool masked = active && tok == mask_id;
  const bool sel = masked && c >= tau;
  uint64_t ballot_sel = __ballot(sel);
  const uint64_t ballot_masked = __ballot(masked);
  bool pick = sel;
  if (ballot_sel == 0 && ballot_masked != 0) {
    // most confident masked position, lowest position on ties
    float bc = masked ? c : -1.f;
    int bi = masked ? i : 0x7fffffff;
    for (int o = 1; o < kWave; o <<= 1) {
      float oc = __shfl_xor(bc, o, kWave);
      int oi = __shfl_xor(bi, o, kWave);
      if (oc > bc || (oc == bc && oi < bi)) { bc = oc; bi = oi; }
    }
    pick = masked && (i == bi);
    ballot_sel = __ballot(pick);
  }
  if (pick) tb[i] = am;
  const int nsel = __popcll(ballot_sel);
  if (i == 0) {
    n_unmasked[b] = nsel;
    remaining[b] = __popcll(ballot_masked) - nsel;
  }
  if (unmasked_idx != nullptr && active) {
    const uint64_t below = ballot_sel & ((1ull << i) - 1ull);
    if (pick) unmasked_idx[b * K + __popcll(below)] = i;
    if (i >= nsel) unmasked_idx[b * K + i] = -1;
  }
}

// Slices of IT * 2048 ids with IT in {1, 2, 4, 8}: about 512 workgroups in total, at
// most kConfMaxSplit slices per row and kConfMaxParts partials per sequence.
ConfPlan conf_plan(int rows, int V, int B) {
  ConfPlan p;
  const int K = rows / (B > 0 ? B : 1);
  const int per = kConfThreads * 8;
  int want = (512 + rows - 1) / rows;  // slices per row for ~512 workgroups
  if (want < 1) want = 1;
  int it = 1;
  while (it < 8 && (int64_t)it * per * want < V) it *= 2;
  int chunk = it * per;
  int ns = (V + chunk - 1) / chunk;
  const int cap = std::min(kConfMaxSplit, kConfMaxParts / (K > 0 ? K : 1));
  if (ns > cap) {  // very large vocabularies: longer slices (looped inside the kernel)
    chunk = ((V + cap - 1) / cap + per - 1) / per * per;
    ns = (V + chunk - 1) / chunk;
  }
  p.it = it;
  p.nsplit = ns;
  p.chunk = chunk;
  p.part_elems = (size_t)rows * ns;
  return p;
}

hipError_t launch_conf_unmask(int ldtype, const ConfPlan& p, const void* logits, int B, int K,
                              int V, int mask_id, float tau, int* tokens, int ld_tokens,
                              float* conf, int* argmax, int* n_unmasked, int* remaining,
                              int* unmasked_idx, float* pm, float* ps, int* pi, hipStream_t st) {
  if (B <= 0 || K <= 0) return hipSuccess;
  if (K > kWave || K * p.nsplit > kConfMaxParts) return hipErrorInvalidValue;
  dim3 grid(p.nsplit, B * K);
#define DLLM_CONF(TT, ITV)                                                                  \
  conf_partials_kernel<TT, ITV><<<grid, kConfThreads, 0, st>>>((const TT*)logits, V, mask_id, \
                                                               p.nsplit, p.chunk, pm, ps, pi)
#define DLLM_CONF_IT(TT)                  \
  switch (p.it) {                         \
    case 1: DLLM_CONF(TT, 1); break;      \
    case 2: DLLM_CONF(TT, 2); break;      \
    case 4: DLLM_CONF(TT, 4); break;      \
    default: DLLM_CONF(TT, 8); break;     \
  }
  if (ldtype == F32) {
    DLLM_CONF_IT(float)
  } else {
    DLLM_CONF_IT(uint16_t)
  }
#undef DLLM_CONF_IT
#undef DLLM_CONF
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  conf_finalize_kernel<<<B, kConfThreads, 0, st>>>(K, p.nsplit, mask_id, tau, pm, ps, pi, tokens,
                                                   ld_tokens, conf, argmax, n_unmasked,
                                                   remaining, unmasked_idx);
  return hipGetLastError();
}

bool lm_conf_fusable(const ConfPlan& p, int V) {
  return V % 8 == 0 && p.chunk == p.it * kConfThreads * 8;
}

hipError_t launch_lm_conf_unmask(const ConfPlan& p, const PartView& pv, const EpiArgs& e,
                                 float* logits, int B, int K, int V, int mask_id, float tau,
                                 int* tokens, int ld_tokens, float* conf, int* argmax,
                                 int* n_unmasked, int* remaining, int* unmasked_idx, float* pm,
                                 float* ps, int* pi, hipStream_t st) {
  if (B <= 0 || K <= 0) return hipSuccess;
  if (K > kWave || K * p.nsplit > kConfMaxParts || !lm_conf_fusable(p, V))
    return hipErrorInvalidValue;
  dim3 grid(p.nsplit, B * K);
  switch (p.it) {
    case 1: lm_conf_partials_kernel<1><<<grid, kConfThreads, 0, st>>>(pv, e, logits, V, mask_id, p.nsplit, p.chunk, pm, ps, pi); break;
    case 2: lm_conf_partials_kernel<2><<<grid, kConfThreads, 0, st>>>(pv, e, logits, V, mask_id, p.nsplit, p.chunk, pm, ps, pi); break;
    case 4: lm_conf_partials_kernel<4><<<grid, kConfThreads, 0, st>>>(pv, e, logits, V, mask_id, p.nsplit, p.chunk, pm, ps, pi); break;
    default: lm_conf_partials_kernel<8><<<grid, kConfThreads, 0, st>>>(pv, e, logits, V, mask_id, p.nsplit, p.chunk, pm, ps, pi); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  conf_finalize_kernel<<<B, kConfThreads, 0, st>>>(K, p.nsplit, mask_id, tau, pm, ps, pi, tokens,
                                                   ld_tokens, conf, argmax, n_unmasked,
                                                   remaining, unmasked_idx);
  return hipGetLastError();
}

}  // namespace dllm
