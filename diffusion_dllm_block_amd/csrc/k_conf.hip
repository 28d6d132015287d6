// Vocab-wide confidence (max softmax probability) and argmax per block row, fused with
// the threshold-unmask compaction of each sequence's block.
//
// Confidence is the probability the model gives its most likely token; every masked
// position of the block at or above the threshold is decoded this step, the others wait
// (ccyt168.com Fast-dLLM article, section 1.2 "Confidence-Aware Parallel Decoding";
// techwalker.com explainer, "Solving the quality loss of parallel decoding").
//
// Layout of the work: grid (nsplit, rows).  Each workgroup streams one slice of one row
// with 16-byte loads and keeps a per-thread online (max, argmax, sum exp) triple; the
// triples are merged in a fixed order (thread-sequential, wave butterfly, waves in
// order) into a per-(row, slice) partial.  The last workgroup of a sequence to finish
// (device-scope arrival counter) merges the slices of its K rows in slice order, one
// lane per row, and runs the unmask rule with wave ballots.  No float atomics: results
// are bit-identical from run to run.
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

__device__ __forceinline__ Trip wave_merge(Trip t) {
  for (int o = 1; o < kWave; o <<= 1) {
    Trip u;
    u.m = __shfl_xor(t.m, o, kWave);
    u.s = __shfl_xor(t.s, o, kWave);
    u.idx = __shfl_xor(t.idx, o, kWave);
    // combine in a lane-independent order: lower lane group first
    bool lower = (threadIdx.x & o) == 0;
    t = lower ? merge(t, u) : merge(u, t);
  }
  return t;
}

template <typename T>
__global__ __launch_bounds__(256) void conf_unmask_kernel(
    const T* __restrict__ logits, int B, int K, int V, int mask_id, float tau, int nsplit,
    int chunk, int* tokens, int ld_tokens, float* conf, int* argmax, int* n_unmasked,
    int* remaining, int* unmasked_idx, float* pm, float* ps, int* pi, int* counters) {
  __shared__ Trip red[4];
  __shared__ int flag;
  const int split = blockIdx.x, row = blockIdx.y;
  const int lo = split * chunk;
  const int hi = min(V, lo + chunk);
  const T* zr = logits + (int64_t)row * V;

  Trip t{-INFINITY, 0.f, 0x7fffffff};
  const bool vec = (V % 8) == 0;  // rows and slices start on 16-byte boundaries
  if (vec) {
    for (int i = lo + threadIdx.x * 8; i < hi; i += blockDim.x * 8) {
      float v[8];
      load8<T>(zr + i, v);
      fold(t, v, 8, i, mask_id);
    }
  } else {
    for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
      float v[8];
      v[0] = Elt<T>::load(zr, i);
      fold(t, v, 1, i, mask_id);
    }
  }
  t = wave_merge(t);
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (lane == 0) red[w] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    Trip a = red[0];
    for (int i = 1; i < (int)(blockDim.x / kWave); ++i) a = merge(a, red[i]);
    int64_t o = (int64_t)row * nsplit + split;
    st_dev(&pm[o], a.m);
    st_dev(&ps[o], a.s);
    st_dev(&pi[o], a.idx);
  }

  const int b = row / K;
  if (!arrive_last(&counters[b], K * nsplit, &flag)) return;
  if (threadIdx.x >= kWave) return;

  // ---- finalize sequence b: lane i handles block position i (K <= 64)
  const int i = lane;
  const bool active = i < K;
  float c = 0.f;
  int am = 0;
  if (active) {
    const int r = b * K + i;
    Trip a{-INFINITY, 0.f, 0x7fffffff};
    for (int sp = 0; sp < nsplit; ++sp) {
      int64_t o = (int64_t)r * nsplit + sp;
      Trip u{ld_dev(&pm[o]), ld_dev(&ps[o]), ld_dev(&pi[o])};
      a = merge(a, u);
    }
    c = 1.0f / a.s;
    am = a.idx;
    conf[r] = c;
    argmax[r] = am;
  }
  int* tb = tokens + (int64_t)b * ld_tokens;
  const int tok = active ? tb[i] : 0;
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
  if (lane == 0) {
    n_unmasked[b] = nsel;
    remaining[b] = __popcll(ballot_masked) - nsel;
  }
  if (unmasked_idx != nullptr && active) {
    const uint64_t below = ballot_sel & ((1ull << lane) - 1ull);
    if (pick) unmasked_idx[b * K + __popcll(below)] = i;
    if (i >= nsel) unmasked_idx[b * K + i] = -1;
  }
}

ConfPlan conf_plan(int rows, int V, int B) {
  ConfPlan p;
  int target = 512;
  int ns = (target + rows - 1) / rows;
  int maxs = (V + 2047) / 2048;  // keep >= 2048 values per slice
  if (ns > maxs) ns = maxs;
  if (ns < 1) ns = 1;
  int chunk = (V + ns - 1) / ns;
  chunk = (chunk + 7) / 8 * 8;
  ns = (V + chunk - 1) / chunk;
  p.nsplit = ns;
  p.chunk = chunk;
  p.part_elems = (size_t)rows * ns;
  p.counters = B;
  return p;
}

hipError_t launch_conf_unmask(int ldtype, const ConfPlan& p, const void* logits, int B, int K,
                              int V, int mask_id, float tau, int* tokens, int ld_tokens,
                              float* conf, int* argmax, int* n_unmasked, int* remaining,
                              int* unmasked_idx, float* pm, float* ps, int* pi, int* counters,
                              hipStream_t st) {
  if (B <= 0 || K <= 0) return hipSuccess;
  dim3 grid(p.nsplit, B * K);
  if (ldtype == F32)
    conf_unmask_kernel<float><<<grid, 256, 0, st>>>(
        (const float*)logits, B, K, V, mask_id, tau, p.nsplit, p.chunk, tokens, ld_tokens, conf,
        argmax, n_unmasked, remaining, unmasked_idx, pm, ps, pi, counters);
  else
    conf_unmask_kernel<uint16_t><<<grid, 256, 0, st>>>(
        (const uint16_t*)logits, B, K, V, mask_id, tau, p.nsplit, p.chunk, tokens, ld_tokens,
        conf, argmax, n_unmasked, remaining, unmasked_idx, pm, ps, pi, counters);
  return hipGetLastError();
}

}  // namespace dllm
