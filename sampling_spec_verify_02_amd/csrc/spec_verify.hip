// Speculative-decoding verification sampler for MI355X (gfx950): kernels and C ABI.
//
// The operation is defined in include/spec_verify.h (accept rule, residual and bonus draws
// from "Speculative Speculative Decoding - асинхронизируй это", SD recap; bonus token from
// "Accélérer Sonar par la Spéculation", section "Décodage spéculatif"; in-order acceptance and
// AL range from "NVIDIA: öt irányelv ...", section "Mit csinál a spekulatív dekódolás?").
//
// Pipeline (all on the caller's stream, no host synchronisation):
//   1. row_stats      one workgroup per (row, 16K-element chunk): exact max and
//                     sum exp((x - max)/T) in fp32 (sampled rows) or max and lowest argmax
//                     (greedy target rows). Streams every needed logit once with 16-byte loads.
//   2. accept_scan    one wavefront per sequence: merges chunk partials, gathers the logits of
//                     the draft tokens, runs the first-reject scan, writes AL and the accepted
//                     tokens, and describes the final draw (residual row j or bonus row L).
//   3. final_norm     fp64 normalisers of the rows of the final draw, per 8K-element chunk.
//   4. final_mass     fp64 per-chunk mass of the draw's weights (residual max(0, p - q), or p).
//   5. final_pick     per sequence: locate the chunk holding u * Z, rescan it with an fp64
//                     prefix scan and write the drawn token.
// The final draw is computed in fp64 because a decision that sits closer to a bin edge than
// ~1e-5 of that bin's width must still agree with an exact computation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "spec_verify.h"

namespace sv {

constexpr int kThreads = 256;          // workgroup size of the streaming kernels (4 waves)
constexpr int kRowChunk = 16384;       // elements per row-statistics unit
constexpr int kFinChunk = 8192;        // elements per final-draw unit
constexpr float kLog2e = 1.4426950408889634f;

enum Mode : int { kNone = 0, kGreedy = 1, kResidual = 2, kBonus = 3 };

struct RowPart {        // partial statistics of one chunk of one row
  float m;              // max of the raw logits in the chunk
  float s;              // sampled rows: sum exp2((x - m) * log2e / T); greedy rows: argmax bits
};

struct SeqDesc {        // what the final draw of one sequence needs
  int mode;             // Mode
  int j;                // position of the final draw
  float mt, md;         // raw maxima of target row j and draft row j
  float u;              // final-draw uniform
  float T;              // temperature
  int pad0, pad1;
};

struct FinPart {        // fp64 normalising sums of one chunk of the final-draw rows
  double st, sd;
};

struct Params {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* lens;
  const float* uniforms;
  const float* temperature;
  int32_t* out_len;
  int32_t* out_tokens;
  int B, D, V;
  int n_row_chunks;
  int n_fin_chunks;
  RowPart* row_part;     // [B][2D+1][n_row_chunks]
  SeqDesc* desc;         // [B]
  FinPart* fin_part;     // [B][n_fin_chunks]
  double* fin_mass;      // [B][n_fin_chunks]
  float* dbg_row_stats;  // optional [B][2D+1][2]
  int32_t* dbg_argmax;   // optional [B][D+1]
  float* dbg_logpq;      // optional [B][D][2]
};

// ------------------------------------------------------------------------------------------
// element access

template <typename E> struct Elem;
template <> struct Elem<uint16_t> {      // bf16 stored as its bit pattern
  static constexpr int kVec = 8;         // elements per 16-byte load
  __device__ static float get(const uint16_t* p, size_t i) {
    return __uint_as_float(uint32_t(p[i]) << 16);
  }
  __device__ static void unpack(const uint4& v, float* x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
};
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float get(const float* p, size_t i) { return p[i]; }
  __device__ static void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
};

__device__ inline bool seq_valid(int L, int D, float T) {
  return L >= 0 && L <= D && isfinite(T) && T >= 0.f;
}

// Row r of sequence b: r in [0, D] is target position r, r in [D+1, 2D] is draft position
// r-D-1. Returns nullptr if the row is not needed.
template <typename E>
__device__ inline const E* row_ptr(const Params& P, int b, int r, int L, bool greedy) {
  if (r <= P.D) {
    if (r > L) return nullptr;
    return static_cast<const E*>(P.target) + (size_t(b) * (P.D + 1) + r) * size_t(P.V);
  }
  const int i = r - P.D - 1;
  if (greedy || i >= L) return nullptr;
  return static_cast<const E*>(P.draft) + (size_t(b) * P.D + i) * size_t(P.V);
}

// ------------------------------------------------------------------------------------------
// reductions

// (m, s) pairs: s is a sum of exp2((x - m) * k). Empty partials carry s == 0.
__device__ inline void ms_combine(float& m, float& s, float m2, float s2, float k) {
  if (s2 == 0.f) return;
  if (s == 0.f) { m = m2; s = s2; return; }
  const float mn = fmaxf(m, m2);
  s = s * __builtin_amdgcn_exp2f((m - mn) * k) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * k);
  m = mn;
}

// (value, index) argmax with the lowest index on ties; index -1 = empty.
__device__ inline void am_combine(float& v, int& i, float v2, int i2) {
  if (i2 < 0) return;
  if (i < 0 || v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ inline void block_reduce_ms(float& m, float& s, float k) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float s2 = __shfl_xor(s, off);
    ms_combine(m, s, m2, s2, k);
  }
  __shared__ float sm[kThreads / 64], ss[kThreads / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[w] = m; ss[w] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k2 = 1; k2 < kThreads / 64; ++k2) ms_combine(m, s, sm[k2], ss[k2], k);
  }
}

__device__ inline void block_reduce_am(float& v, int& i) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float v2 = __shfl_xor(v, off);
    const int i2 = __shfl_xor(i, off);
    am_combine(v, i, v2, i2);
  }
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sv[w] = v; si[w] = i; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kThreads / 64; ++k) am_combine(v, i, sv[k], si[k]);
  }
}

__device__ inline double block_sum_f64(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  __shared__ double sd[kThreads / 64];
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sd[w] = x;
  __syncthreads();
  double t = 0.0;
  for (int k = 0; k < kThreads / 64; ++k) t += sd[k];
  return t;   // identical in every thread
}

// ------------------------------------------------------------------------------------------
// 1. row statistics

template <typename E>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(Params P) {
  constexpr int kVec = Elem<E>::kVec;
  constexpr int kPerThread = kRowChunk / kVec / kThreads;   // 16-byte loads per thread
  const int R = 2 * P.D + 1;
  const int unit = blockIdx.x;
  const int c = unit % P.n_row_chunks;
  const int br = unit / P.n_row_chunks;
  const int b = br / R, r = br % R;
  const int L = P.lens ? P.lens[b] : P.D;
  const float T = P.temperature[b];
  if (!seq_valid(L, P.D, T)) return;
  const bool greedy = (T == 0.f);
  const E* row = row_ptr<E>(P, b, r, L, greedy);
  if (row == nullptr) return;

  const size_t c0 = size_t(c) * kRowChunk;
  const int n = int(min(size_t(kRowChunk), size_t(P.V) - c0));
  const E* p = row + c0;
  const bool aligned = (reinterpret_cast<uintptr_t>(p) & 15) == 0;
  const int nvec = aligned ? n / kVec : 0;
  const int tid = threadIdx.x;
  RowPart* out = P.row_part + size_t(br) * P.n_row_chunks + c;

  uint4 buf[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int vi = tid + k * kThreads;
    if (vi < nvec) buf[k] = reinterpret_cast<const uint4*>(p)[vi];
  }

  if (greedy) {
    float best = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int vi = tid + k * kThreads;
      if (vi < nvec) {
        float x[kVec];
        Elem<E>::unpack(buf[k], x);
#pragma unroll
        for (int e = 0; e < kVec; ++e)
          if (bi < 0 || x[e] > best) { best = x[e]; bi = vi * kVec + e; }
      }
    }
    for (int i = nvec * kVec + tid; i < n; i += kThreads)
      am_combine(best, bi, Elem<E>::get(p, i), i);
    block_reduce_am(best, bi);
    if (tid == 0) { out->m = best; out->s = __int_as_float(bi < 0 ? -1 : int(c0) + bi); }
    return;
  }

  const float k2 = kLog2e / T;
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int vi = tid + k * kThreads;
    if (vi < nvec) {
      float x[kVec];
      Elem<E>::unpack(buf[k], x);
#pragma unroll
      for (int e = 0; e < kVec; ++e) m = fmaxf(m, x[e]);
    }
  }
  for (int i = nvec * kVec + tid; i < n; i += kThreads) m = fmaxf(m, Elem<E>::get(p, i));
  float s = 0.f;
  if (m > -INFINITY) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int vi = tid + k * kThreads;
      if (vi < nvec) {
        float x[kVec];
        Elem<E>::unpack(buf[k], x);
#pragma unroll
        for (int e = 0; e < kVec; ++e) s += __builtin_amdgcn_exp2f((x[e] - m) * k2);
      }
    }
    for (int i = nvec * kVec + tid; i < n; i += kThreads)
      s += __builtin_amdgcn_exp2f((Elem<E>::get(p, i) - m) * k2);
  }
  block_reduce_ms(m, s, k2);
  if (tid == 0) { out->m = m; out->s = s; }
}

// ------------------------------------------------------------------------------------------
// 2. accept scan: one wavefront per sequence

template <typename E>
__global__ __launch_bounds__(64) void accept_scan_kernel(Params P) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int D = P.D, R = 2 * D + 1;
  const int L = P.lens ? P.lens[b] : D;
  const float T = P.temperature[b];
  int32_t* toks = P.out_tokens + size_t(b) * (D + 1);
  SeqDesc* desc = P.desc + b;

  bool ok = seq_valid(L, D, T);
  if (ok) {
    bool bad = false;
    for (int i = lane; i < L; i += 64) {
      const int x = P.tokens[size_t(b) * D + i];
      bad |= (x < 0 || x >= P.V);
    }
    ok = !__any(bad);
  }
  if (P.dbg_row_stats)
    for (int r = lane; r < R; r += 64) {
      P.dbg_row_stats[(size_t(b) * R + r) * 2] = NAN;
      P.dbg_row_stats[(size_t(b) * R + r) * 2 + 1] = NAN;
    }
  if (P.dbg_argmax)
    for (int i = lane; i <= D; i += 64) P.dbg_argmax[size_t(b) * (D + 1) + i] = -1;
  if (P.dbg_logpq)
    for (int i = lane; i < 2 * D; i += 64) P.dbg_logpq[size_t(b) * D * 2 + i] = NAN;
  if (!ok) {
    for (int i = lane; i <= D; i += 64) toks[i] = -1;
    if (lane == 0) { P.out_len[b] = 0; desc->mode = kNone; }
    return;
  }
  const bool greedy = (T == 0.f);

  __shared__ float s_m[2 * SV_MAX_D + 1];
  __shared__ float s_lns[2 * SV_MAX_D + 1];
  __shared__ int s_arg[SV_MAX_D + 1];
  const float k2 = greedy ? 0.f : kLog2e / T;
  for (int r = lane; r < R; r += 64) {
    if (row_ptr<E>(P, b, r, L, greedy) == nullptr) continue;
    const RowPart* part = P.row_part + (size_t(b) * R + r) * P.n_row_chunks;
    if (greedy) {
      float v = -INFINITY;
      int idx = -1;
      for (int c = 0; c < P.n_row_chunks; ++c) am_combine(v, idx, part[c].m, __float_as_int(part[c].s));
      s_arg[r] = idx;
      if (P.dbg_argmax) P.dbg_argmax[size_t(b) * (D + 1) + r] = idx;
    } else {
      float m = -INFINITY, s = 0.f;
      for (int c = 0; c < P.n_row_chunks; ++c) ms_combine(m, s, part[c].m, part[c].s, k2);
      s_m[r] = m;
      s_lns[r] = logf(s);
      if (P.dbg_row_stats) {
        P.dbg_row_stats[(size_t(b) * R + r) * 2] = m / T;
        P.dbg_row_stats[(size_t(b) * R + r) * 2 + 1] = logf(s);
      }
    }
  }
  __syncthreads();

  if (greedy) {
    if (lane == 0) {
      int j = 0;
      while (j < L && P.tokens[size_t(b) * D + j] == s_arg[j]) { toks[j] = s_arg[j]; ++j; }
      toks[j] = s_arg[j];
      for (int i = j + 1; i <= D; ++i) toks[i] = -1;
      P.out_len[b] = j + 1;
      desc->mode = kGreedy;
      desc->j = j;
    }
    return;
  }

  // sampled: log-domain ratio per tested position, then first rejection
  bool reject = false;
  int x = 0;
  if (lane < L) {
    x = P.tokens[size_t(b) * D + lane];
    const E* trow = static_cast<const E*>(P.target) + (size_t(b) * (D + 1) + lane) * size_t(P.V);
    const E* drow = static_cast<const E*>(P.draft) + (size_t(b) * D + lane) * size_t(P.V);
    const float xt = Elem<E>::get(trow, x);
    const float xd = Elem<E>::get(drow, x);
    const float lp = (xt - s_m[lane]) / T - s_lns[lane];
    const float lq = (xd - s_m[D + 1 + lane]) / T - s_lns[D + 1 + lane];
    const float ratio = expf(lp - lq);
    const float u = P.uniforms[size_t(b) * (D + 1) + lane];
    reject = !(u < fminf(1.f, ratio));
    if (P.dbg_logpq) {
      P.dbg_logpq[(size_t(b) * D + lane) * 2] = lp;
      P.dbg_logpq[(size_t(b) * D + lane) * 2 + 1] = lq;
    }
  }
  const unsigned long long rej = __ballot(reject);
  const int j = rej ? __builtin_ctzll(rej) : L;
  for (int i = lane; i <= D; i += 64) {
    if (i < j) toks[i] = P.tokens[size_t(b) * D + i];
    else toks[i] = -1;
  }
  if (lane == 0) {
    P.out_len[b] = j + 1;
    desc->mode = (j < L) ? kResidual : kBonus;
    desc->j = j;
    desc->mt = s_m[j];
    desc->md = (j < L) ? s_m[D + 1 + j] : 0.f;
    desc->u = P.uniforms[size_t(b) * (D + 1) + D];
    desc->T = T;
  }
}

// ------------------------------------------------------------------------------------------
// 3-5. final draw in fp64

template <typename E>
__device__ inline double exp_weight(const E* row, int v, double m, double invT) {
  return exp((double(Elem<E>::get(row, v)) - m) * invT);
}

template <typename E>
__global__ __launch_bounds__(kThreads) void final_norm_kernel(Params P) {
  const int b = blockIdx.x / P.n_fin_chunks;
  const int c = blockIdx.x % P.n_fin_chunks;
  const SeqDesc d = P.desc[b];
  if (d.mode != kResidual && d.mode != kBonus) return;
  const E* trow = static_cast<const E*>(P.target) + (size_t(b) * (P.D + 1) + d.j) * size_t(P.V);
  const E* drow = static_cast<const E*>(P.draft) + (size_t(b) * P.D + d.j) * size_t(P.V);
  const double invT = 1.0 / double(d.T);
  const int v0 = c * kFinChunk, v1 = min(P.V, v0 + kFinChunk);
  double st = 0.0, sd = 0.0;
  for (int v = v0 + threadIdx.x; v < v1; v += kThreads) {
    st += exp_weight(trow, v, double(d.mt), invT);
    if (d.mode == kResidual) sd += exp_weight(drow, v, double(d.md), invT);
  }
  st = block_sum_f64(st);
  sd = block_sum_f64(sd);
  if (threadIdx.x == 0) P.fin_part[size_t(b) * P.n_fin_chunks + c] = FinPart{st, sd};
}

__device__ inline void final_totals(const Params& P, int b, double& st, double& sd) {
  st = 0.0;
  sd = 0.0;
  const FinPart* fp = P.fin_part + size_t(b) * P.n_fin_chunks;
  for (int c = 0; c < P.n_fin_chunks; ++c) { st += fp[c].st; sd += fp[c].sd; }
}

template <typename E>
__device__ inline double residual_weight(const E* trow, const E* drow, int v, const SeqDesc& d,
                                         double invT, double it, double id) {
  const double pt = exp_weight(trow, v, double(d.mt), invT) * it;
  const double pd = exp_weight(drow, v, double(d.md), invT) * id;
  return fmax(0.0, pt - pd);
}

template <typename E>
__global__ __launch_bounds__(kThreads) void final_mass_kernel(Params P) {
  const int b = blockIdx.x / P.n_fin_chunks;
  const int c = blockIdx.x % P.n_fin_chunks;
  const SeqDesc d = P.desc[b];
  if (d.mode != kResidual) return;
  double st, sd;
  final_totals(P, b, st, sd);
  const double it = 1.0 / st, id = 1.0 / sd, invT = 1.0 / double(d.T);
  const E* trow = static_cast<const E*>(P.target) + (size_t(b) * (P.D + 1) + d.j) * size_t(P.V);
  const E* drow = static_cast<const E*>(P.draft) + (size_t(b) * P.D + d.j) * size_t(P.V);
  const int v0 = c * kFinChunk, v1 = min(P.V, v0 + kFinChunk);
  double w = 0.0;
  for (int v = v0 + threadIdx.x; v < v1; v += kThreads) w += residual_weight(trow, drow, v, d, invT, it, id);
  w = block_sum_f64(w);
  if (threadIdx.x == 0) P.fin_mass[size_t(b) * P.n_fin_chunks + c] = w;
}

template <typename E>
__global__ __launch_bounds__(kThreads) void final_pick_kernel(Params P) {
  const int b = blockIdx.x;
  const SeqDesc d = P.desc[b];
  if (d.mode != kResidual && d.mode != kBonus) return;
  const int tid = threadIdx.x;
  const int nF = P.n_fin_chunks;
  double st, sd;
  final_totals(P, b, st, sd);
  const double it = 1.0 / st, id = 1.0 / sd, invT = 1.0 / double(d.T);
  const E* trow = static_cast<const E*>(P.target) + (size_t(b) * (P.D + 1) + d.j) * size_t(P.V);
  const E* drow = static_cast<const E*>(P.draft) + (size_t(b) * P.D + d.j) * size_t(P.V);

  // residual weights, or (bonus, or a residual of zero total mass) the target's exp weights
  bool residual = (d.mode == kResidual);
  const double* mass = P.fin_mass + size_t(b) * nF;
  const FinPart* fp = P.fin_part + size_t(b) * nF;
  __shared__ int s_chunk;
  __shared__ int s_last;
  __shared__ double s_rem;
  __shared__ int s_residual;
  if (tid == 0) {
    double Z = 0.0;
    if (residual) for (int c = 0; c < nF; ++c) Z += mass[c];
    if (!(Z > 0.0)) { residual = false; Z = 0.0; for (int c = 0; c < nF; ++c) Z += fp[c].st; }
    const double t = double(d.u) * Z;
    double pre = 0.0;
    int cs = -1, lastpos = -1;
    double rem = 0.0;
    for (int c = 0; c < nF; ++c) {
      const double wc = residual ? mass[c] : fp[c].st;
      if (wc > 0.0) lastpos = c;
      if (cs < 0 && pre + wc > t) { cs = c; rem = t - pre; }
      pre += wc;
    }
    s_last = (cs < 0) ? 1 : 0;
    s_chunk = (cs < 0) ? lastpos : cs;
    s_rem = rem;
    s_residual = residual ? 1 : 0;
  }
  __syncthreads();
  residual = s_residual != 0;
  const int c = s_chunk;
  if (c < 0) {                          // no positive weight at all (non-finite logits)
    if (tid == 0) P.out_tokens[size_t(b) * (P.D + 1) + d.j] = -1;
    return;
  }
  const double rem = s_rem;
  const int v0 = c * kFinChunk, v1 = min(P.V, v0 + kFinChunk);
  const int n = v1 - v0;
  const int per = (n + kThreads - 1) / kThreads;
  const int a0 = v0 + tid * per, a1 = min(v1, a0 + per);
  auto weight = [&](int v) {
    return residual ? residual_weight(trow, drow, v, d, invT, it, id)
                    : exp_weight(trow, v, double(d.mt), invT);
  };
  double ts = 0.0;
  int my_last = -1;
  for (int v = a0; v < a1; ++v) {
    const double w = weight(v);
    ts += w;
    if (w > 0.0) my_last = v;
  }
  // exclusive prefix of the per-thread sums (Hillis-Steele in LDS)
  __shared__ double s_scan[kThreads];
  __shared__ int s_found;
  __shared__ int s_lastv[kThreads];
  s_scan[tid] = ts;
  s_lastv[tid] = my_last;
  if (tid == 0) s_found = -1;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const double add = (tid >= off) ? s_scan[tid - off] : 0.0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  // thread t owns [incl_{t-1}, incl_t): consecutive stored values, so exactly one owner
  const double pre = (tid > 0) ? s_scan[tid - 1] : 0.0;
  if (!s_last && ts > 0.0 && pre <= rem && rem < s_scan[tid]) {
    double acc = pre;
    int k = my_last;
    for (int v = a0; v < a1; ++v) {
      acc += weight(v);
      if (acc > rem) { k = v; break; }
    }
    s_found = k;
  }
  __syncthreads();
  if (tid == 0) {
    int k = s_found;
    if (k < 0) {                        // rounding put u*Z past the end: last positive weight
      for (int t2 = kThreads - 1; t2 >= 0 && k < 0; --t2) k = s_lastv[t2];
    }
    P.out_tokens[size_t(b) * (P.D + 1) + d.j] = k;
  }
}

// ------------------------------------------------------------------------------------------
// host side

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  int n_row_chunks, n_fin_chunks;
  size_t off_row, off_desc, off_fin, off_mass, total;
};

inline bool make_layout(int B, int D, int V, Layout& L) {
  if (B <= 0 || D < 0 || V <= 0 || D > SV_MAX_D) return false;
  L.n_row_chunks = (V + kRowChunk - 1) / kRowChunk;
  L.n_fin_chunks = (V + kFinChunk - 1) / kFinChunk;
  const size_t R = size_t(2) * D + 1;
  L.off_row = 0;
  L.off_desc = align256(size_t(B) * R * L.n_row_chunks * sizeof(RowPart));
  L.off_fin = L.off_desc + align256(size_t(B) * sizeof(SeqDesc));
  L.off_mass = L.off_fin + align256(size_t(B) * L.n_fin_chunks * sizeof(FinPart));
  L.total = L.off_mass + align256(size_t(B) * L.n_fin_chunks * sizeof(double));
  return true;
}

struct DeviceWorkspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};

std::mutex g_ws_mutex;
std::vector<DeviceWorkspace> g_ws;

// Optional timing of the row-statistics kernel: when armed, each call records one event pair
// around that kernel on the caller's stream.
struct Profile {
  std::vector<hipEvent_t> begin, end;
  int used = 0;
  bool armed = false;
};
std::mutex g_prof_mutex;
Profile g_prof;

int check_args(const void* t, const void* d, const int32_t* tok, const float* u, const float* temp,
               int32_t* ol, int32_t* ot, int B, int D, int V) {
  if (B <= 0 || D < 0 || V <= 0 || D > SV_MAX_D) return SV_EINVAL;
  if (!t || !u || !temp || !ol || !ot) return SV_EINVAL;
  if (D > 0 && (!d || !tok)) return SV_EINVAL;
  // element counts must fit comfortably in 64-bit byte offsets
  const unsigned __int128 n = (unsigned __int128)B * (unsigned __int128)(D + 1) * (unsigned __int128)V;
  if (n > ((unsigned __int128)1 << 60)) return SV_EINVAL;
  return SV_OK;
}

template <typename E>
int launch_all(Params& P, hipStream_t stream) {
  const int R = 2 * P.D + 1;
  const size_t n_units = size_t(P.B) * R * P.n_row_chunks;
  if (n_units > 0x7fffffffull) return SV_EINVAL;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  {
    std::lock_guard<std::mutex> g(g_prof_mutex);
    if (g_prof.armed && g_prof.used < int(g_prof.begin.size())) {
      ev0 = g_prof.begin[size_t(g_prof.used)];
      ev1 = g_prof.end[size_t(g_prof.used)];
      ++g_prof.used;
    }
  }
  if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return SV_EHIP;
  hipLaunchKernelGGL(row_stats_kernel<E>, dim3(unsigned(n_units)), dim3(kThreads), 0, stream, P);
  if (ev1 && hipEventRecord(ev1, stream) != hipSuccess) return SV_EHIP;
  hipLaunchKernelGGL(accept_scan_kernel<E>, dim3(P.B), dim3(64), 0, stream, P);
  const unsigned n_fin = unsigned(size_t(P.B) * P.n_fin_chunks);
  hipLaunchKernelGGL(final_norm_kernel<E>, dim3(n_fin), dim3(kThreads), 0, stream, P);
  hipLaunchKernelGGL(final_mass_kernel<E>, dim3(n_fin), dim3(kThreads), 0, stream, P);
  hipLaunchKernelGGL(final_pick_kernel<E>, dim3(P.B), dim3(kThreads), 0, stream, P);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

int run(int dtype, const void* target, const void* draft, const int32_t* tokens,
        const int32_t* lens, const float* uniforms, int B, int D, int V, const float* temperature,
        int32_t* out_len, int32_t* out_tokens, void* ws, size_t ws_bytes, float* dbg_stats,
        int32_t* dbg_argmax, float* dbg_logpq, hipStream_t stream) {
  if (dtype != 0 && dtype != 1) return SV_EDTYPE;
  int rc = check_args(target, draft, tokens, uniforms, temperature, out_len, out_tokens, B, D, V);
  if (rc != SV_OK) return rc;
  Layout lay;
  make_layout(B, D, V, lay);

  std::unique_lock<std::mutex> lock(g_ws_mutex, std::defer_lock);
  if (ws == nullptr) {
    int dev = 0, count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return SV_ENODEV;
    if (hipGetDevice(&dev) != hipSuccess) return SV_ENODEV;
    lock.lock();
    if (g_ws.size() <= size_t(dev)) g_ws.resize(size_t(dev) + 1);
    DeviceWorkspace& w = g_ws[size_t(dev)];
    if (w.bytes < lay.total) {
      if (w.ptr) {
        // the old buffer may still be in use by enqueued work on any stream
        if (hipDeviceSynchronize() != hipSuccess) return SV_EHIP;
        (void)hipFree(w.ptr);
        w.ptr = nullptr;
        w.bytes = 0;
      }
      if (hipMalloc(&w.ptr, lay.total) != hipSuccess) return SV_ENOMEM;
      w.bytes = lay.total;
    }
    ws = w.ptr;
    ws_bytes = w.bytes;
  } else {
    if (ws_bytes < lay.total || (reinterpret_cast<uintptr_t>(ws) & 255)) return SV_ENOMEM;
  }

  Params P;
  P.target = target;
  P.draft = draft;
  P.tokens = tokens;
  P.lens = lens;
  P.uniforms = uniforms;
  P.temperature = temperature;
  P.out_len = out_len;
  P.out_tokens = out_tokens;
  P.B = B;
  P.D = D;
  P.V = V;
  P.n_row_chunks = lay.n_row_chunks;
  P.n_fin_chunks = lay.n_fin_chunks;
  char* base = static_cast<char*>(ws);
  P.row_part = reinterpret_cast<RowPart*>(base + lay.off_row);
  P.desc = reinterpret_cast<SeqDesc*>(base + lay.off_desc);
  P.fin_part = reinterpret_cast<FinPart*>(base + lay.off_fin);
  P.fin_mass = reinterpret_cast<double*>(base + lay.off_mass);
  P.dbg_row_stats = dbg_stats;
  P.dbg_argmax = dbg_argmax;
  P.dbg_logpq = dbg_logpq;
  return dtype == 1 ? launch_all<uint16_t>(P, stream) : launch_all<float>(P, stream);
}

}  // namespace sv

extern "C" {

int spec_verify_bf16(const void* target_logits, const void* draft_logits,
                     const int32_t* draft_tokens, const int32_t* draft_lens,
                     const float* uniforms, int B, int D, int V, const float* temperature,
                     int32_t* out_accept_len, int32_t* out_tokens, hipStream_t stream) {
  return sv::run(1, target_logits, draft_logits, draft_tokens, draft_lens, uniforms, B, D, V,
                 temperature, out_accept_len, out_tokens, nullptr, 0, nullptr, nullptr, nullptr,
                 stream);
}

int spec_verify_f32(const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const int32_t* draft_lens,
                    const float* uniforms, int B, int D, int V, const float* temperature,
                    int32_t* out_accept_len, int32_t* out_tokens, hipStream_t stream) {
  return sv::run(0, target_logits, draft_logits, draft_tokens, draft_lens, uniforms, B, D, V,
                 temperature, out_accept_len, out_tokens, nullptr, 0, nullptr, nullptr, nullptr,
                 stream);
}

size_t spec_verify_workspace_bytes(int B, int D, int V) {
  sv::Layout lay;
  return sv::make_layout(B, D, V, lay) ? lay.total : 0;
}

int spec_verify_ws(int dtype, const void* target_logits, const void* draft_logits,
                   const int32_t* draft_tokens, const int32_t* draft_lens,
                   const float* uniforms, int B, int D, int V, const float* temperature,
                   int32_t* out_accept_len, int32_t* out_tokens, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  if (workspace == nullptr) return SV_EINVAL;
  return sv::run(dtype, target_logits, draft_logits, draft_tokens, draft_lens, uniforms, B, D,
                 V, temperature, out_accept_len, out_tokens, workspace, workspace_bytes, nullptr,
                 nullptr, nullptr, stream);
}

int spec_verify_debug(int dtype, const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const int32_t* draft_lens,
                      const float* uniforms, int B, int D, int V, const float* temperature,
                      int32_t* out_accept_len, int32_t* out_tokens, float* row_stats,
                      int32_t* row_argmax, float* logpq_x, hipStream_t stream) {
  return sv::run(dtype, target_logits, draft_logits, draft_tokens, draft_lens, uniforms, B, D,
                 V, temperature, out_accept_len, out_tokens, nullptr, 0, row_stats, row_argmax,
                 logpq_x, stream);
}

const char* spec_verify_strerror(int code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument";
    case SV_EDTYPE: return "unknown dtype";
    case SV_EHIP: return "HIP runtime error";
    case SV_ENODEV: return "no usable GPU device";
    case SV_ENOMEM: return "workspace allocation failed or workspace too small";
    default: return "unknown status";
  }
}

int spec_verify_version(void) { return 100; }

int spec_verify_profile_start(int max_calls) {
  if (max_calls <= 0 || max_calls > (1 << 20)) return SV_EINVAL;
  std::lock_guard<std::mutex> g(sv::g_prof_mutex);
  if (sv::g_prof.armed) return SV_EINVAL;
  sv::g_prof.begin.assign(size_t(max_calls), nullptr);
  sv::g_prof.end.assign(size_t(max_calls), nullptr);
  for (int i = 0; i < max_calls; ++i) {
    if (hipEventCreate(&sv::g_prof.begin[size_t(i)]) != hipSuccess ||
        hipEventCreate(&sv::g_prof.end[size_t(i)]) != hipSuccess)
      return SV_EHIP;
  }
  sv::g_prof.used = 0;
  sv::g_prof.armed = true;
  return SV_OK;
}

int spec_verify_profile_stop(float* out_ms, int max_out, int* n_recorded) {
  std::lock_guard<std::mutex> g(sv::g_prof_mutex);
  if (!sv::g_prof.armed) return SV_EINVAL;
  int rc = SV_OK;
  const int n = sv::g_prof.used;
  for (int i = 0; i < n; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(sv::g_prof.end[size_t(i)]) != hipSuccess ||
        hipEventElapsedTime(&ms, sv::g_prof.begin[size_t(i)], sv::g_prof.end[size_t(i)]) !=
            hipSuccess)
      rc = SV_EHIP;
    if (out_ms && i < max_out) out_ms[i] = ms;
  }
  if (n_recorded) *n_recorded = n;
  for (auto e : sv::g_prof.begin) if (e) (void)hipEventDestroy(e);
  for (auto e : sv::g_prof.end) if (e) (void)hipEventDestroy(e);
  sv::g_prof = sv::Profile();
  return rc;
}

}  // extern "C"
