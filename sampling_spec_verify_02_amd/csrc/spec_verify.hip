// Speculative-decoding verification sampler for MI355X (gfx950): fused kernel and C ABI.
//
// The operation is the one stated in include/spec_verify.h: accept / reject / residual rule
// from "Speculative Speculative Decoding - асинхронизируй это" (recap of standard speculative
// decoding), the bonus token from "Accélérer Sonar par la Spéculation" (section "Décodage
// spéculatif"), in-order acceptance up to the first mismatch and AL in [1, 1 + D] from
// "NVIDIA: öt irányelv ..." (section "Mit csinál a spekulatív dekódolás?").
//
// One kernel per call, with two kinds of workgroups.
//
// * Row workgroups (one-shot, one per 32 KB chunk of a row, position-major order: all position-0
//   rows of the batch first, then position 1, ...). Each streams its chunk with non-temporal
//   16-byte loads and produces the chunk's exact max and fp32 sum exp((x - max) / T) (sampled
//   rows) or max and lowest argmax (greedy target rows); the chunk holding the draft token x_p
//   also records the logit at x_p. Rows the method does not need (padding, draft rows of greedy
//   sequences) cost no memory traffic. The workgroup completing the last chunk of a (sequence,
//   position) pair evaluates that position's test on its own, u_p < min(1, p_p(x_p)/q_p(x_p))
//   (or x_p == argmax for greedy), and ORs "position p done" and "position p rejects" into the
//   sequence's 64-bit state word. The outcome is decided once a rejection is preceded by a
//   complete prefix of evaluated positions, or once positions 0..L are all done without one;
//   exactly one OR makes that transition, and its workgroup writes the accepted tokens and AL
//   and queues the sequence's final draw. Most sequences are decided after their first few
//   positions, long before the streaming of later positions ends.
// * Worker workgroups (a few per CU, persistent) take final-draw items from the queue. Item
//   (b, f) evaluates a 2048-element chunk of the final row(s) in fp64 (target and draft row j
//   after a rejection at j, target row L for the bonus draw): fp64 normalising sums, and the
//   residual mass linearised around the fp32 estimate rho~ of rho = S_t / S_d (elements whose
//   ln(e_t / e_d) is clearly above ln rho~ are certainly in the positive part of p - q and
//   contribute e_t / S_t - e_d / S_d, those clearly below contribute nothing, those inside the
//   band are summed apart with the range of their x_t - x_d: one value means one exact ratio
//   class, resolved exactly later). The worker completing a sequence's last item picks the
//   token: exact normalisers, exact chunk masses, the chunk holding u * Z, and an fp64
//   prefix-scan rescan of that chunk.
//
// Nothing on the row path ever waits for another workgroup. Hand-offs use device-coherent
// (sc1) atomic stores and loads and relaxed device-scope atomics: a device-scope
// release/acquire fence would write back and invalidate the XCD's whole L2 on every hand-off.
// The counters come in two sets used by alternate calls; each call clears the set the next
// call will use, so no workgroup has to wait for the others to finish.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "spec_verify.h"

namespace sv {

constexpr int kThreads = 256;                 // workgroup size (4 wavefronts)
constexpr int kWaves = kThreads / 64;
constexpr int kRowChunkBytes = 32768;         // bytes of one row per row workgroup
constexpr int kRowVecs = kRowChunkBytes / 16 / kThreads;   // 16-byte loads per thread (8)
constexpr int kFinPer = 8;                    // consecutive elements per lane and block
constexpr int kMinFinChunk = 2048;            // smallest final-draw item (elements)
constexpr int kMaxFinChunk = 32768;           // largest final-draw item (elements)
constexpr bool kConcurrent = false;           // final-draw kernel alongside the row kernel
constexpr int kWorkersPerCU = kConcurrent ? 1 : 4;   // final-draw workgroups per CU
constexpr float kLog2e = 1.4426950408889634f;
// Half-width of the band (in ln(e_t/e_d)) inside which an element's sign in max(0, p - q) is
// not decided from the fp32 estimate of ln(S_t/S_d). The fp32 statistics are accurate to a
// few 1e-6, so the exact ln(S_t/S_d) lies well inside; the pick checks that it does.
constexpr double kBand = 3e-5;
constexpr long long kSpinLimit = 4000000;     // polls before a wait gives up

enum Mode : int { kNone = 0, kGreedy = 1, kResidual = 2, kBonus = 3 };

struct RowPart {      // partial statistics of one row chunk
  float m;            // max of the raw logits in the chunk
  float s;            // sampled rows: sum exp((x - m) / T); greedy rows: bits of the argmax
  float xv;           // logit at the draft token of this position, if it lies in the chunk
  float pad;
};

struct PosInfo {      // what the evaluation of one (sequence, position) found
  float mt, md;       // exact row maxima (target, draft)
  float lnrho;        // fp32 ln(S_t / S_d)
  int g;              // greedy: target argmax
};

struct SeqDesc {      // what the final draw of one sequence needs
  int mode;           // Mode
  int j;              // position of the final draw
  float mt, md;       // exact maxima of target row j and draft row j
  float lnrho;        // fp32 estimate of ln(S_t / S_d) for row j (residual only)
  float u;            // final-draw uniform
  float T;            // temperature
  float pad;
};

struct FinPart {      // fp64 sums of one final-draw chunk
  double st, sd;      // sum e_t, sum e_d   (e = exp((x - max) / T))
  double at, ad;      // sums over elements certainly in the positive part of p - q
  double bt, bd;      // sums over the elements inside the band
  double dmin, dmax;  // min / max of x_t - x_d inside the band (+inf / -inf: none)
};

struct Hdr {          // per-call counters of one set
  unsigned q_seq;     // sequences queued for a final draw
  unsigned q_items;   // final-draw items published
  unsigned q_claim;   // final-draw items claimed by workers
  unsigned decided;   // sequences whose outcome is decided (and queued if sampled)
  unsigned pad[60];
};

struct CounterSet {   // everything that must be zero when a call starts
  Hdr* hdr;
  unsigned long long* st;   // [B] done bits 0..31, reject bits 32..63
  unsigned* pc;             // [B][D+1] completed chunks of the position's rows
  unsigned* fdone;          // [B] completed final-draw items
  unsigned* qs;             // [B] queue slots: sequence + 1 (0 = not yet written)
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
  int R;              // rows per sequence, 2D + 1 (target 0..D, then draft 0..D-1)
  int rch;            // elements per row chunk
  int nchunk;         // row chunks per row
  int fch;            // elements per final-draw item (multiple of 512)
  int nF;             // final-draw items per sequence
  int n_workers;      // worker workgroups (blockIdx < n_workers)
  CounterSet cur;     // this call's counters
  CounterSet nxt;     // the next call's counters, cleared by the workers
  RowPart* rpart;     // [B][R][nchunk]
  PosInfo* pinfo;     // [B][D+1]
  SeqDesc* desc;      // [B]
  FinPart* fpart;     // [B][nF]
  double* fmass;      // [B][nF] scratch of the pick
  float* dbg_row_stats;  // optional [B][R][2]
  int32_t* dbg_argmax;   // optional [B][D+1]
  float* dbg_logpq;      // optional [B][D][2]
};

// ------------------------------------------------------------------------------------------
// device-coherent accesses

template <typename T>
__device__ inline void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ inline T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned add_dev(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned long long or_dev(unsigned long long* p, unsigned long long v) {
  return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wavefront's earlier vector-memory operations (the device-coherent stores of
// a result) have completed, before a counter announces them.
__device__ inline void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------------------------------------
// element access

template <typename E> struct Elem;
template <> struct Elem<uint16_t> {          // bf16 bit patterns
  static constexpr int kVec = 8;             // elements per 16-byte load
  __device__ static float get(const uint16_t* p, size_t i) {
    return __uint_as_float(uint32_t(p[i]) << 16);
  }
  __device__ static float lane(const uint4& v, int e) {
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float get(const float* p, size_t i) { return p[i]; }
  __device__ static float lane(const uint4& v, int e) {
    return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
  }
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The run p[a .. a+n), n <= kFinPer, zero past n, kept packed as loaded (16-byte loads when
// aligned; element loads otherwise, packed the same way).
template <typename E> struct Run;
template <> struct Run<uint16_t> {
  uint32_t w[4];
  __device__ void load(const uint16_t* p, int a, int n) {
    const uint16_t* q = p + a;
    if (n == kFinPer && (reinterpret_cast<uintptr_t>(q) & 15) == 0) {
      const uint4 v = *reinterpret_cast<const uint4*>(q);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = (2 * k < n) ? q[2 * k] : 0u;
        const uint32_t hi = (2 * k + 1 < n) ? q[2 * k + 1] : 0u;
        w[k] = lo | (hi << 16);
      }
    }
  }
  __device__ float at(int e) const {
    return __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
  }
};
template <> struct Run<float> {
  float x[kFinPer];
  __device__ void load(const float* p, int a, int n) {
    const float* q = p + a;
    if (n == kFinPer && (reinterpret_cast<uintptr_t>(q) & 15) == 0) {
      const float4 v0 = reinterpret_cast<const float4*>(q)[0];
      const float4 v1 = reinterpret_cast<const float4*>(q)[1];
      x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
      x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
    } else {
#pragma unroll
      for (int e = 0; e < kFinPer; ++e) x[e] = (e < n) ? q[e] : 0.f;
    }
  }
  __device__ float at(int e) const { return x[e]; }
};

// wave-uniform values kept in scalar registers
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline double uniform(double v) {
  const unsigned long long u = __double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readfirstlane(unsigned(u));
  const unsigned hi = __builtin_amdgcn_readfirstlane(unsigned(u >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ inline bool seq_valid(int L, int D, float T) {
  return L >= 0 && L <= D && isfinite(T) && T >= 0.f;
}

// chunks of the rows of (sequence, position p) that the method needs
__device__ inline int pair_chunks(int p, int L, bool greedy, int nchunk) {
  return (p <= L ? nchunk : 0) + ((!greedy && p < L) ? nchunk : 0);
}

// Has the outcome been decided by state word w? Sets j (position of the final token).
__device__ inline bool decided(unsigned long long w, int L, int& j) {
  const unsigned done = unsigned(w), rej = unsigned(w >> 32);
  const int k = __builtin_ctz(~done);                 // positions 0..k-1 evaluated
  const unsigned pre = (k >= 32) ? 0xffffffffu : ((1u << k) - 1u);
  const unsigned r = rej & pre;
  if (r) { j = __builtin_ctz(r); return true; }
  if (k >= L + 1) { j = L; return true; }
  return false;
}

// ------------------------------------------------------------------------------------------
// reductions (fixed trees, so identical inputs give identical bits)

// (m, s) pairs: s is a sum of exp2((x - m) * k); empty partials carry s == 0.
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

__device__ inline void wave_ms(float& m, float& s, float k) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float s2 = __shfl_xor(s, off);
    ms_combine(m, s, m2, s2, k);
  }
}

__device__ inline void wave_am(float& v, int& i) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float v2 = __shfl_xor(v, off);
    const int i2 = __shfl_xor(i, off);
    am_combine(v, i, v2, i2);
  }
}

__device__ inline double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}
__device__ inline double wave_min(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmin(x, __shfl_xor(x, off));
  return x;
}
__device__ inline double wave_max(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmax(x, __shfl_xor(x, off));
  return x;
}

// ------------------------------------------------------------------------------------------
// shared memory of one workgroup

struct Shared {
  double exp_tab[256];          // 2^(i/256), workers only
  double red[kWaves][8];
  int flag;
};

// fp64 exp: e^t = 2^(k/256) * e^f with k = rint(t * 256 / ln 2) and f = t - k * ln2/256
// (|f| <= ln2/512; ln2/256 split in two parts so that k * hi is exact), e^f from its degree-4
// Taylor polynomial (truncation below 4e-17 relative), 2^(k/256) = tab[k mod 256] * 2^(k div 256).
__device__ inline double exp64(double t, const double* tab) {
  const double y = t * 369.3299304675746;                  // 256 / ln 2
  const double kf = __builtin_rint(y);
  double f = fma(-kf, 0.002707606172407395, t);            // ln2/256, high part
  f = fma(-kf, 1.6548911585192516e-12, f);                 // ln2/256, low part
  const int k = int(kf);
  const double p = fma(fma(fma(fma(f, 1.0 / 24.0, 1.0 / 6.0), f, 0.5), f, 1.0), f, 1.0);
  return ldexp(tab[k & 255] * p, k >> 8);
}

// ------------------------------------------------------------------------------------------
// outcome of a sequence (wavefront 0 of the deciding workgroup)

template <typename E>
__device__ void decide(const Params& P, int b, int L, float T, bool greedy, int j, int lane) {
  const int D = P.D;
  const int32_t* xs = P.tokens + size_t(b) * D;
  int32_t* toks = P.out_tokens + size_t(b) * (D + 1);
  const bool bad = lane < L && (xs[lane] < 0 || xs[lane] >= P.V);   // L <= D <= 31
  if (__any(bad)) {
    for (int i = lane; i <= D; i += 64) toks[i] = -1;
    if (lane == 0) {
      P.out_len[b] = 0;
      add_dev(&P.cur.hdr->decided, 1u);
    }
    return;
  }
  if (greedy) {
    for (int i = lane; i <= D; i += 64)
      toks[i] = (i <= j) ? ld_dev(&P.pinfo[size_t(b) * (D + 1) + i].g) : -1;
    if (lane == 0) {
      P.out_len[b] = j + 1;
      add_dev(&P.cur.hdr->decided, 1u);
    }
    return;
  }
  for (int i = lane; i <= D; i += 64) {
    if (i < j) toks[i] = xs[i];
    else if (i > j) toks[i] = -1;      // position j is written by the final draw
  }
  if (lane == 0) {
    P.out_len[b] = j + 1;
    const PosInfo* pi = P.pinfo + size_t(b) * (D + 1) + j;
    SeqDesc* d = P.desc + b;
    st_dev(&d->mode, int(j < L ? kResidual : kBonus));
    st_dev(&d->j, j);
    st_dev(&d->mt, ld_dev(&pi->mt));
    st_dev(&d->md, j < L ? ld_dev(&pi->md) : 0.f);
    st_dev(&d->lnrho, j < L ? ld_dev(&pi->lnrho) : 0.f);
    st_dev(&d->u, P.uniforms[size_t(b) * (D + 1) + D]);
    st_dev(&d->T, T);
    wait_stores();
    const unsigned slot = add_dev(&P.cur.hdr->q_seq, 1u);
    st_dev(P.cur.qs + slot, unsigned(b + 1));
    wait_stores();
    add_dev(&P.cur.hdr->q_items, unsigned(P.nF));
    add_dev(&P.cur.hdr->decided, 1u);
  }
}

// Evaluation of position p of sequence b once all its chunks are in (whole workgroup calls it;
// wavefront 0 does the work).
template <typename E>
__device__ void evaluate(const Params& P, int b, int p, int L, float T, bool greedy, int tid) {
  if (tid >= 64) return;
  const int lane = tid;
  const int D = P.D, R = P.R, nc = P.nchunk;
  const RowPart* tpart = P.rpart + (size_t(b) * R + p) * nc;
  const RowPart* dpart = P.rpart + (size_t(b) * R + D + 1 + p) * nc;
  PosInfo* pi = P.pinfo + size_t(b) * (D + 1) + p;
  bool reject = false;
  if (greedy) {
    float v = -INFINITY;
    int idx = -1;
    for (int c = lane; c < nc; c += 64)
      am_combine(v, idx, ld_dev(&tpart[c].m), __float_as_int(ld_dev(&tpart[c].s)));
    wave_am(v, idx);
    if (p < L) reject = (P.tokens[size_t(b) * D + p] != idx);
    if (lane == 0) {
      st_dev(&pi->g, idx);
      if (P.dbg_argmax) P.dbg_argmax[size_t(b) * (D + 1) + p] = idx;
    }
  } else {
    const float k2 = kLog2e / T;
    float mt = -INFINITY, stt = 0.f, md = -INFINITY, sd = 0.f;
    for (int c = lane; c < nc; c += 64) {
      ms_combine(mt, stt, ld_dev(&tpart[c].m), ld_dev(&tpart[c].s), k2);
      if (p < L) ms_combine(md, sd, ld_dev(&dpart[c].m), ld_dev(&dpart[c].s), k2);
    }
    wave_ms(mt, stt, k2);
    if (p < L) wave_ms(md, sd, k2);
    const float lnt = logf(stt), lnd = logf(sd);
    float lp = NAN, lq = NAN;
    if (p < L) {
      const int x = P.tokens[size_t(b) * D + p];
      if (x >= 0 && x < P.V) {
        const int cx = x / P.rch;
        const float xt = ld_dev(&tpart[cx].xv);
        const float xd = ld_dev(&dpart[cx].xv);
        lp = (xt - mt) / T - lnt;
        lq = (xd - md) / T - lnd;
        const float ratio = expf(lp - lq);
        reject = !(P.uniforms[size_t(b) * (D + 1) + p] < fminf(1.f, ratio));
      } else {
        reject = true;                 // invalid token: the decision marks the row
      }
    }
    if (lane == 0) {
      st_dev(&pi->mt, mt);
      st_dev(&pi->md, md);
      st_dev(&pi->lnrho, lnt - lnd);
      if (P.dbg_row_stats) {
        P.dbg_row_stats[(size_t(b) * R + p) * 2] = mt / T;
        P.dbg_row_stats[(size_t(b) * R + p) * 2 + 1] = lnt;
        if (p < L) {
          P.dbg_row_stats[(size_t(b) * R + D + 1 + p) * 2] = md / T;
          P.dbg_row_stats[(size_t(b) * R + D + 1 + p) * 2 + 1] = lnd;
        }
      }
      if (P.dbg_logpq && p < L) {
        P.dbg_logpq[(size_t(b) * D + p) * 2] = lp;
        P.dbg_logpq[(size_t(b) * D + p) * 2 + 1] = lq;
      }
    }
  }
  unsigned long long old = 0;
  if (lane == 0) {
    wait_stores();
    const unsigned long long bits = (1ull << p) | (reject ? (1ull << (32 + p)) : 0ull);
    old = or_dev(P.cur.st + b, bits);
    const unsigned long long now = old | bits;
    int j0 = 0, j1 = 0;
    const bool was = decided(old, L, j0);
    const bool is = decided(now, L, j1);
    old = (is && !was) ? (unsigned long long)(j1 + 1) : 0ull;
  }
  old = __shfl(old, 0);
  if (old) decide<E>(P, b, L, T, greedy, int(old) - 1, lane);
}

// ------------------------------------------------------------------------------------------
// row workgroup

template <typename E>
__device__ void row_workgroup(const Params& P, Shared& sm, long long rid, int tid) {
  constexpr int kV = Elem<E>::kVec;
  const int nc = P.nchunk;
  const long long per_p = (long long)P.B * 2 * nc;
  const int p = int(rid / per_p);
  const long long rem = rid - (long long)p * per_p;
  const int b = int(rem / (2 * nc));
  const int which = int(rem % (2 * nc)) / nc;          // 0 target row p, 1 draft row p
  const int c = int(rem % nc);
  const int D = P.D;
  const int L = P.lens ? P.lens[b] : D;
  const float T = P.temperature[b];

  if (!seq_valid(L, D, T)) {
    // invalid length or temperature: one workgroup of the sequence marks the row
    if (p == 0 && which == 0 && c == 0) {
      int32_t* toks = P.out_tokens + size_t(b) * (D + 1);
      for (int i = tid; i <= D; i += kThreads) toks[i] = -1;
      if (tid == 0) {
        P.out_len[b] = 0;
        add_dev(&P.cur.hdr->decided, 1u);
      }
    }
    return;
  }
  const bool greedy = (T == 0.f);
  if (which == 0 ? (p > L) : (greedy || p >= L)) return;   // row not needed

  const int r = which == 0 ? p : D + 1 + p;
  const E* row = which == 0
      ? static_cast<const E*>(P.target) + (size_t(b) * (D + 1) + p) * size_t(P.V)
      : static_cast<const E*>(P.draft) + (size_t(b) * D + p) * size_t(P.V);
  const int c0 = c * P.rch;
  const int n = min(P.rch, P.V - c0);
  const E* ptr = row + c0;
  const bool aligned = (reinterpret_cast<uintptr_t>(ptr) & 15) == 0;
  const int nvec = aligned ? n / kV : 0;

  uint4 buf[kRowVecs];
#pragma unroll
  for (int k = 0; k < kRowVecs; ++k) {
    const int vi = tid + k * kThreads;
    if (vi < nvec) buf[k] = load_stream(reinterpret_cast<const uint4*>(ptr) + vi);
  }
  float xv = 0.f;
  if (!greedy && tid == 0 && p < L) {
    const int x = P.tokens[size_t(b) * D + p];
    if (x >= c0 && x < c0 + n) xv = Elem<E>::get(row, x);
  }

  float m, s;
  if (greedy) {
    float best = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int k = 0; k < kRowVecs; ++k) {
      const int vi = tid + k * kThreads;
      if (vi < nvec) {
#pragma unroll
        for (int e = 0; e < kV; ++e) {
          const float x = Elem<E>::lane(buf[k], e);
          if (bi < 0 || x > best) { best = x; bi = vi * kV + e; }
        }
      }
    }
    for (int i = nvec * kV + tid; i < n; i += kThreads) am_combine(best, bi, Elem<E>::get(ptr, i), i);
    wave_am(best, bi);
    float* rv = reinterpret_cast<float*>(&sm.red[0][0]);
    int* ri = reinterpret_cast<int*>(&sm.red[0][4]);
    if ((tid & 63) == 0) { rv[tid >> 6] = best; ri[tid >> 6] = bi; }
    __syncthreads();
    if (tid == 0)
      for (int w = 1; w < kWaves; ++w) am_combine(best, bi, rv[w], ri[w]);
    m = best;
    s = __int_as_float(bi < 0 ? -1 : c0 + bi);
  } else {
    // online max / sum per 16-byte vector: only one vector's elements are live at a time
    const float k2 = kLog2e / T;
    float mx = -INFINITY, sum = 0.f;
#pragma unroll
    for (int k = 0; k < kRowVecs; ++k) {
      const int vi = tid + k * kThreads;
      if (vi < nvec) {
        float mk = Elem<E>::lane(buf[k], 0);
#pragma unroll
        for (int e = 1; e < kV; ++e) mk = fmaxf(mk, Elem<E>::lane(buf[k], e));
        if (k == 0) {
          mx = mk;
        } else {
          const float mn = fmaxf(mx, mk);
          sum *= __builtin_amdgcn_exp2f((mx - mn) * k2);
          mx = mn;
        }
        const float off = -mx * k2;
#pragma unroll
        for (int e = 0; e < kV; ++e) sum += __builtin_amdgcn_exp2f(fmaf(Elem<E>::lane(buf[k], e), k2, off));
      }
    }
    for (int i = nvec * kV + tid; i < n; i += kThreads) {
      const float x = Elem<E>::get(ptr, i);
      if (x > mx) {
        sum = (sum == 0.f) ? 0.f : sum * __builtin_amdgcn_exp2f((mx - x) * k2);
        mx = x;
      }
      sum += __builtin_amdgcn_exp2f((x - mx) * k2);
    }
    wave_ms(mx, sum, k2);
    float* rm = reinterpret_cast<float*>(&sm.red[0][0]);
    float* rs = reinterpret_cast<float*>(&sm.red[0][4]);
    if ((tid & 63) == 0) { rm[tid >> 6] = mx; rs[tid >> 6] = sum; }
    __syncthreads();
    if (tid == 0)
      for (int w = 1; w < kWaves; ++w) ms_combine(mx, sum, rm[w], rs[w], k2);
    m = mx;
    s = sum;
  }

  if (tid == 0) {
    RowPart* out = P.rpart + (size_t(b) * P.R + r) * nc + c;
    st_dev(&out->m, m);
    st_dev(&out->s, s);
    st_dev(&out->xv, xv);
    wait_stores();
    const unsigned done = add_dev(P.cur.pc + size_t(b) * (D + 1) + p, 1u) + 1u;
    sm.flag = (done == unsigned(pair_chunks(p, L, greedy, nc))) ? 1 : 0;
  }
  __syncthreads();
  if (sm.flag) evaluate<E>(P, b, p, L, T, greedy, tid);
}

// ------------------------------------------------------------------------------------------
// final draw (wave-level workers)
//
// A final-draw item covers fch consecutive elements (fch a multiple of 512) of the final row(s)
// of one sequence. Inside an item, block k holds elements [512k, 512k + 512) and lane l of the
// wavefront handles elements 512k + 8l .. 512k + 8l + 7 of each block (16-byte loads).

struct Draw {           // what the fp64 evaluation of one sequence's final row(s) needs
  bool residual;
  int j;
  double mt, md, invT, lnrho, u;
};

template <typename E>
__device__ inline const E* final_row(const Params& P, int b, int j, bool draft) {
  return draft ? static_cast<const E*>(P.draft) + (size_t(b) * P.D + j) * size_t(P.V)
               : static_cast<const E*>(P.target) + (size_t(b) * (P.D + 1) + j) * size_t(P.V);
}

// Exact weight of element e of the runs: e_t when target_only, else max(0, e_t/S_t - e_d/S_d).
template <typename E>
__device__ inline double exact_weight(const Run<E>& rt, const Run<E>& rd, int e, const Draw& w,
                                      bool target_only, double it, double id, const double* tab) {
  const double et = exp64((double(rt.at(e)) - w.mt) * w.invT, tab);
  if (target_only) return et;
  const double ed = exp64((double(rd.at(e)) - w.md) * w.invT, tab);
  return fmax(0.0, et * it - ed * id);
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ inline double wave_inclusive_scan(double x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Sum of the exact weights of one item's elements (fixed order); target_only as above.
template <typename E>
__device__ inline double item_exact_mass(const Params& P, const E* trow, const E* drow,
                                         const Draw& w, int f, bool target_only, double it,
                                         double id, const double* tab, int lane) {
  const int a0 = f * P.fch;
  const int nblk = (min(P.fch, P.V - a0) + 511) / 512;
  double s = 0.0;
  for (int k = 0; k < nblk; ++k) {
    const int a = a0 + 512 * k + 8 * lane;
    const int n = max(0, min(kFinPer, P.V - a));
    if (n > 0) {
      Run<E> rt, rd;
      rt.load(trow, a, n);
      if (!target_only) rd.load(drow, a, n);
#pragma unroll
      for (int e = 0; e < kFinPer; ++e) {
        if (e < n) s += exact_weight<E>(rt, rd, e, w, target_only, it, id, tab);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  return wave_sum(s);
}

// The last final-draw item of a sequence: exact normalisers, item masses, token (one wavefront).
template <typename E>
__device__ void wave_pick(const Params& P, const double* tab, int b, const Draw& w, int lane) {
  const int nF = P.nF;
  const FinPart* fp = P.fpart + size_t(b) * nF;
  double* mass = P.fmass + size_t(b) * nF;
  const E* trow = final_row<E>(P, b, w.j, false);
  const E* drow = w.residual ? final_row<E>(P, b, w.j, true) : trow;

  double st = 0.0, sd = 0.0;
  int multi = 0;
  for (int f = lane; f < nF; f += 64) {
    st += ld_dev(&fp[f].st);
    sd += ld_dev(&fp[f].sd);
    if (ld_dev(&fp[f].dmin) < ld_dev(&fp[f].dmax)) multi = 1;
  }
  st = wave_sum(st);
  sd = wave_sum(sd);
  const double it = 1.0 / st, id = 1.0 / sd;
  // did the band hold the exact ratio, and is every item's in-band set one ratio class?
  const bool slow = w.residual && (__any(multi) || !(fabs(log(st / sd) - w.lnrho) < kBand));

  bool target_only = !w.residual;
  if (!slow) {
    for (int f = lane; f < nF; f += 64) {
      double m;
      if (target_only) {
        m = ld_dev(&fp[f].st);
      } else {
        m = ld_dev(&fp[f].at) * it - ld_dev(&fp[f].ad) * id;
        if (ld_dev(&fp[f].dmin) <= ld_dev(&fp[f].dmax))            // one in-band ratio class
          m += fmax(0.0, ld_dev(&fp[f].bt) * it - ld_dev(&fp[f].bd) * id);
        m = fmax(0.0, m);
      }
      st_dev(mass + f, m);
    }
  } else {
    for (int f = 0; f < nF; ++f) {
      const double m = item_exact_mass<E>(P, trow, drow, w, f, false, it, id, tab, lane);
      if (lane == 0) st_dev(mass + f, m);
    }
  }
  wait_stores();

  // inclusive prefix of the item masses (64 at a time); Z is the last prefix
  auto prefix = [&](bool from_st) {
    double total = 0.0;
    for (int base = 0; base < nF; base += 64) {
      const int f = base + lane;
      const double v = (f < nF) ? (from_st ? ld_dev(&fp[f].st) : ld_dev(mass + f)) : 0.0;
      const double inc = wave_inclusive_scan(v, lane) + total;
      if (f < nF) st_dev(mass + f, inc);
      total = __shfl(inc, 63);
    }
    wait_stores();
    return total;
  };
  double total = prefix(false);
  if (!(total > 0.0) && !target_only) {
    target_only = true;                // residual of zero mass (rounding only): draw from p_j
    total = prefix(true);
  }
  const double t = w.u * total;

  // first item whose inclusive prefix exceeds t (else the last item with positive mass)
  int fstar = nF, flast = -1;
  for (int base = 0; base < nF; base += 64) {
    const int f = base + lane;
    const double inc = (f < nF) ? ld_dev(mass + f) : 0.0;
    const double prev = (f > 0 && f < nF) ? ld_dev(mass + f - 1) : 0.0;
    const unsigned long long over = __ballot(f < nF && inc > t);
    const unsigned long long pos = __ballot(f < nF && inc > prev);
    if (over && fstar == nF) fstar = base + __builtin_ctzll(over);
    if (pos) flast = base + 63 - __builtin_clzll(pos);
  }
  const bool past_end = (fstar >= nF);
  if (past_end) fstar = flast;
  int32_t* out = P.out_tokens + size_t(b) * (P.D + 1) + w.j;
  if (fstar < 0) {                     // no positive weight at all
    if (lane == 0) *out = -1;
    return;
  }
  double run = (fstar > 0) ? ld_dev(mass + fstar - 1) : 0.0;

  // rescan the chosen item block by block, in ascending element order
  const int a0 = fstar * P.fch;
  const int nblk = (min(P.fch, P.V - a0) + 511) / 512;
  int found = -1, last_pos = -1;
  for (int k = 0; k < nblk && found < 0; ++k) {
    const int a = a0 + 512 * k + 8 * lane;
    const int n = max(0, min(kFinPer, P.V - a));
    Run<E> rt, rd;
    double ls = 0.0;
    int my_last = -1;
    if (n > 0) {
      rt.load(trow, a, n);
      if (!target_only) rd.load(drow, a, n);
#pragma unroll
      for (int e = 0; e < kFinPer; ++e) {
        if (e < n) {
          const double wt = exact_weight<E>(rt, rd, e, w, target_only, it, id, tab);
          ls += wt;
          if (wt > 0.0) my_last = a + e;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const double inc = wave_inclusive_scan(ls, lane) + run;
    const double pre = inc - ls;
    // lane l owns [prefix before l, prefix through l): consecutive stored values, one owner
    const double lo = __shfl_up(inc, 1);
    const double mylo = (lane == 0) ? run : lo;
    last_pos = max(last_pos, my_last);
    const bool owner = !past_end && ls > 0.0 && mylo <= t && t < inc;
    (void)pre;
    const unsigned long long own = __ballot(owner);
    if (own) {
      const int ol = __builtin_ctzll(own);
      int k2 = -1;
      if (lane == ol) {
        double acc = mylo;
#pragma unroll
        for (int e = 0; e < kFinPer; ++e) {
          if (e < n && k2 < 0) {
            acc += exact_weight<E>(rt, rd, e, w, target_only, it, id, tab);
            if (acc > t) k2 = a + e;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (k2 < 0) k2 = my_last;
      }
      found = __shfl(k2, ol);
    }
    run = __shfl(inc, 63);
  }
  // rounding put u * Z past the end: the last element with positive weight
  for (int off = 32; off > 0; off >>= 1) last_pos = max(last_pos, __shfl_xor(last_pos, off));
  if (lane == 0) *out = (found >= 0) ? found : last_pos;
}

template <typename E>
__device__ void wave_fin_item(const Params& P, const double* tab, int b, int f, const Draw& w,
                              int lane) {
  const E* trow = final_row<E>(P, b, w.j, false);
  const E* drow = w.residual ? final_row<E>(P, b, w.j, true) : trow;
  const int a0 = f * P.fch;
  const int nblk = (min(P.fch, P.V - a0) + 511) / 512;
  const double hi = w.lnrho + kBand, lo = w.lnrho - kBand;
  double st = 0, sd = 0, at = 0, ad = 0, bt = 0, bd = 0, dmin = INFINITY, dmax = -INFINITY;
  for (int k = 0; k < nblk; ++k) {
    const int a = a0 + 512 * k + 8 * lane;
    const int n = max(0, min(kFinPer, P.V - a));
    if (n <= 0) continue;
    Run<E> rt, rd;
    rt.load(trow, a, n);
    if (w.residual) rd.load(drow, a, n);
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) {
      if (e >= n) continue;
      const double xt = double(rt.at(e));
      const double tt = (xt - w.mt) * w.invT;
      const double et = exp64(tt, tab);
      st += et;
      if (w.residual) {
        const double xd = double(rd.at(e));
        const double td = (xd - w.md) * w.invT;
        const double ed = exp64(td, tab);
        sd += ed;
        const double l = tt - td;                      // ln(e_t / e_d)
        if (l > hi) {
          at += et;
          ad += ed;
        } else if (l >= lo) {
          bt += et;
          bd += ed;
          dmin = fmin(dmin, xt - xd);
          dmax = fmax(dmax, xt - xd);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one element at a time: bounded register use
    }
  }
  st = wave_sum(st);
  sd = wave_sum(sd);
  at = wave_sum(at);
  ad = wave_sum(ad);
  bt = wave_sum(bt);
  bd = wave_sum(bd);
  dmin = wave_min(dmin);
  dmax = wave_max(dmax);
  int last = 0;
  if (lane == 0) {
    FinPart* out = P.fpart + size_t(b) * P.nF + f;
    st_dev(&out->st, st);
    st_dev(&out->sd, sd);
    st_dev(&out->at, at);
    st_dev(&out->ad, ad);
    st_dev(&out->bt, bt);
    st_dev(&out->bd, bd);
    st_dev(&out->dmin, dmin);
    st_dev(&out->dmax, dmax);
    wait_stores();
    last = (add_dev(P.cur.fdone + b, 1u) + 1u == unsigned(P.nF)) ? 1 : 0;
  }
  last = __shfl(last, 0);
  if (last) wave_pick<E>(P, tab, b, w, lane);
}

// One worker wavefront. Wavefront gw owns the queue items gw, gw + W, gw + 2W, ... (W = all
// worker wavefronts) and takes them in that order, waiting for each to be published when the
// final-draw kernel runs alongside the row kernel. It stops at the first owned item that can
// no longer appear (every sequence decided and the item beyond the last published one).
template <typename E>
__device__ void wave_worker(const Params& P, const double* tab, int gw, int lane) {
  const unsigned nF = unsigned(P.nF);
  const unsigned W = unsigned(P.n_workers) * kWaves;
  int cur_b = -1;
  Draw w = {};
  for (unsigned u = unsigned(gw);; u += W) {
    int b = -1;
    if (lane == 0) {
      long long spins = 0;
      bool go = false;
      for (;;) {
        if (u < ld_dev(&P.cur.hdr->q_items)) { go = true; break; }
        if (ld_dev(&P.cur.hdr->decided) >= unsigned(P.B) && u >= ld_dev(&P.cur.hdr->q_items)) break;
        if (++spins > kSpinLimit) break;               // never expected: give up, do not hang
        __builtin_amdgcn_s_sleep(8);
      }
      if (go) {
        const unsigned slot = u / nF;
        unsigned q = 0;
        for (spins = 0; (q = ld_dev(P.cur.qs + slot)) == 0u && spins < kSpinLimit; ++spins)
          __builtin_amdgcn_s_sleep(1);
        b = int(q) - 1;
      }
    }
    b = uniform(__shfl(b, 0));
    if (b < 0) break;
    const int f = int(u % nF);
    if (b != cur_b) {                  // descriptor fields, one per lane, in one round trip
      const SeqDesc* d = P.desc + b;
      int iv = 0;
      float fv = 0.f;
      if (lane == 0) iv = ld_dev(&d->mode);
      if (lane == 1) iv = ld_dev(&d->j);
      if (lane == 2) fv = ld_dev(&d->mt);
      if (lane == 3) fv = ld_dev(&d->md);
      if (lane == 4) fv = ld_dev(&d->lnrho);
      if (lane == 5) fv = ld_dev(&d->u);
      if (lane == 6) fv = ld_dev(&d->T);
      w.residual = uniform(__shfl(iv, 0)) == kResidual;
      w.j = uniform(__shfl(iv, 1));
      w.mt = uniform(double(__shfl(fv, 2)));
      w.md = uniform(double(__shfl(fv, 3)));
      w.lnrho = uniform(double(__shfl(fv, 4)));
      w.u = uniform(double(__shfl(fv, 5)));
      w.invT = uniform(1.0 / double(__shfl(fv, 6)));
      cur_b = b;
    }
    wave_fin_item<E>(P, tab, b, f, w, lane);
  }
}

template <typename E>
__device__ void worker(const Params& P, Shared& sm, int wid, int tid) {
  for (int i = tid; i < 256; i += kThreads) sm.exp_tab[i] = exp2(double(i) / 256.0);

  // clear the counters of the next call (no workgroup of this call touches them)
  {
    const long long stride = (long long)P.n_workers * kThreads;
    const long long me = (long long)wid * kThreads + tid;
    for (long long i = me; i < P.B; i += stride) {
      st_dev(P.nxt.st + i, 0ull);
      st_dev(P.nxt.fdone + i, 0u);
      st_dev(P.nxt.qs + i, 0u);
    }
    const long long npc = (long long)P.B * (P.D + 1);
    for (long long i = me; i < npc; i += stride) st_dev(P.nxt.pc + i, 0u);
    if (wid == 0 && tid < 4) st_dev(reinterpret_cast<unsigned*>(P.nxt.hdr) + tid, 0u);
  }
  __syncthreads();
  wave_worker<E>(P, sm.exp_tab, wid * kWaves + (tid >> 6), tid & 63);
}

// ------------------------------------------------------------------------------------------
// the kernel

// Row kernel: one workgroup per row chunk (its own register budget, so many stay resident).
template <typename E>
__global__ __launch_bounds__(kThreads) void row_kernel(Params P) {
  __shared__ Shared sm;
  row_workgroup<E>(P, sm, (long long)blockIdx.x, threadIdx.x);
}

// Final-draw kernel: persistent worker workgroups (four worker wavefronts each).
template <typename E>
__global__ __launch_bounds__(kThreads) void final_kernel(Params P) {
  __shared__ Shared sm;
  worker<E>(P, sm, int(blockIdx.x), threadIdx.x);
}

// Clears the counter region (when a workspace meets a new B or D).
__global__ void clear_kernel(unsigned* p, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ------------------------------------------------------------------------------------------
// host side

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: [counter set 0][counter set 1] [row partials][position info][descriptors]
//            [final-draw partials][pick scratch]. A counter set is [Hdr][st B][pc B(D+1)]
//            [fdone B][qs B]; both sets must be zero when a workspace is first used.
struct Layout {
  int rch, nchunk, nF;
  size_t set_bytes, off_st, off_pc, off_fdone, off_qs;   // within a counter set
  size_t off_rpart, off_pinfo, off_desc, off_fpart, off_fmass, total;
};

inline bool make_layout(int B, int D, int V, int elem_bytes, Layout& L) {
  if (B <= 0 || D < 0 || V <= 0 || D > SV_MAX_D) return false;
  L.rch = kRowChunkBytes / elem_bytes;
  L.nchunk = int((size_t(V) + L.rch - 1) / L.rch);
  L.nF = int((size_t(V) + kMinFinChunk - 1) / kMinFinChunk);   // most items a row can need
  size_t o = align256(sizeof(Hdr));
  L.off_st = o;    o += align256(size_t(B) * 8);
  L.off_pc = o;    o += align256(size_t(B) * (D + 1) * 4);
  L.off_fdone = o; o += align256(size_t(B) * 4);
  L.off_qs = o;    o += align256(size_t(B) * 4);
  L.set_bytes = o;
  o = 2 * L.set_bytes;
  const size_t R = size_t(2) * D + 1;
  L.off_rpart = o; o += align256(size_t(B) * R * L.nchunk * sizeof(RowPart));
  L.off_pinfo = o; o += align256(size_t(B) * (D + 1) * sizeof(PosInfo));
  L.off_desc = o;  o += align256(size_t(B) * sizeof(SeqDesc));
  L.off_fpart = o; o += align256(size_t(B) * L.nF * sizeof(FinPart));
  L.off_fmass = o; o += align256(size_t(B) * L.nF * sizeof(double));
  L.total = o;
  return true;
}

// Workspace bytes: the larger of the two dtypes' layouts, so one size serves both.
inline size_t workspace_bytes(int B, int D, int V) {
  Layout a, b;
  if (!make_layout(B, D, V, 2, a) || !make_layout(B, D, V, 4, b)) return 0;
  return a.total > b.total ? a.total : b.total;
}

inline CounterSet counter_set(char* base, const Layout& L, int k) {
  char* s = base + size_t(k) * L.set_bytes;
  CounterSet c;
  c.hdr = reinterpret_cast<Hdr*>(s);
  c.st = reinterpret_cast<unsigned long long*>(s + L.off_st);
  c.pc = reinterpret_cast<unsigned*>(s + L.off_pc);
  c.fdone = reinterpret_cast<unsigned*>(s + L.off_fdone);
  c.qs = reinterpret_cast<unsigned*>(s + L.off_qs);
  return c;
}

struct DeviceWorkspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};

struct WsState {      // host-side knowledge about one workspace
  long long calls = 0;        // calls made with it (the parity picks the counter set)
  int B = -1, D = -1;         // counter layout of the last call (-1: zero-filled, unused)
};

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, DeviceWorkspace> g_ws;   // library buffers per stream
std::map<void*, WsState> g_ws_state;

struct Profile {        // optional timing of the kernel: one event pair per call
  std::vector<hipEvent_t> begin, end;
  int used = 0;
  bool armed = false;
};
std::mutex g_prof_mutex;
Profile g_prof;

std::mutex g_dev_mutex;
std::map<int, int> g_cus;        // device -> compute units

// A second stream per (device, caller stream) for the final-draw workers, with the two events
// that fork it from and join it back to the caller's stream. Default priority.
struct Side {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mutex;
std::map<std::pair<int, hipStream_t>, Side> g_side;

Side* side_stream(hipStream_t caller) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_side_mutex);
  Side& sd = g_side[{dev, caller}];
  if (!sd.s) {
    if (hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking) != hipSuccess) { sd.s = nullptr; return nullptr; }
    if (hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&sd.join, hipEventDisableTiming) != hipSuccess)
      return nullptr;
  }
  return &sd;
}

int check_args(const void* t, const void* d, const int32_t* tok, const float* u, const float* temp,
               int32_t* ol, int32_t* ot, int B, int D, int V) {
  if (B <= 0 || D < 0 || V <= 0 || D > SV_MAX_D) return SV_EINVAL;
  if (!t || !u || !temp || !ol || !ot) return SV_EINVAL;
  if (D > 0 && (!d || !tok)) return SV_EINVAL;
  const unsigned __int128 n = (unsigned __int128)B * (unsigned __int128)(D + 1) * (unsigned __int128)V;
  if (n > ((unsigned __int128)1 << 60)) return SV_EINVAL;
  return SV_OK;
}

int compute_units(int dev) {
  std::lock_guard<std::mutex> lk(g_dev_mutex);
  auto it = g_cus.find(dev);
  if (it != g_cus.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  g_cus[dev] = cus;
  return cus;
}

template <typename E>
int launch(Params& P, int dev, hipStream_t stream) {
  const int cus = compute_units(dev);
  if (cus <= 0) return SV_EHIP;
  // Worker wavefronts: four per workgroup, kWorkersPerCU workgroups per CU. Items are sized so
  // each worker wavefront gets about four: small items keep the work after the last decision
  // short, large ones keep the per-item overhead low when there are many draws.
  const long long waves = 4ll * kWorkersPerCU * cus;
  long long fch = ((long long)P.B * P.V + 4 * waves - 1) / (4 * waves);
  fch = (fch + 511) / 512 * 512;
  fch = fch < kMinFinChunk ? kMinFinChunk : (fch > kMaxFinChunk ? kMaxFinChunk : fch);
  P.fch = int(fch);
  P.nF = int((P.V + fch - 1) / fch);
  const long long items = (long long)P.B * P.nF;
  const long long wg = (items + 3) / 4;
  P.n_workers = int(wg < (long long)kWorkersPerCU * cus ? wg : (long long)kWorkersPerCU * cus);
  const long long rows = (long long)(P.D + 1) * P.B * 2 * P.nchunk;
  if (rows > 0x7fffffffll) return SV_EINVAL;

  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  {
    std::lock_guard<std::mutex> g(g_prof_mutex);
    if (g_prof.armed && g_prof.used < int(g_prof.begin.size())) {
      ev0 = g_prof.begin[size_t(g_prof.used)];
      ev1 = g_prof.end[size_t(g_prof.used)];
      ++g_prof.used;
    }
  }
  if (kConcurrent) {
    // the final-draw workers run alongside the row kernel on a second stream: fork after the
    // caller's earlier work, join before the caller's later work
    Side* side = side_stream(stream);
    if (!side) return SV_EHIP;
    if (hipEventRecord(side->fork, stream) != hipSuccess) return SV_EHIP;
    if (hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess) return SV_EHIP;
    hipLaunchKernelGGL(final_kernel<E>, dim3(unsigned(P.n_workers)), dim3(kThreads), 0, side->s, P);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
    if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return SV_EHIP;
    hipLaunchKernelGGL(row_kernel<E>, dim3(unsigned(rows)), dim3(kThreads), 0, stream, P);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
    if (ev1 && hipEventRecord(ev1, stream) != hipSuccess) return SV_EHIP;
    if (hipEventRecord(side->join, side->s) != hipSuccess) return SV_EHIP;
    if (hipStreamWaitEvent(stream, side->join, 0) != hipSuccess) return SV_EHIP;
    return SV_OK;
  }
  if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return SV_EHIP;
  hipLaunchKernelGGL(row_kernel<E>, dim3(unsigned(rows)), dim3(kThreads), 0, stream, P);
  if (hipGetLastError() != hipSuccess) return SV_EHIP;
  if (ev1 && hipEventRecord(ev1, stream) != hipSuccess) return SV_EHIP;
  hipLaunchKernelGGL(final_kernel<E>, dim3(unsigned(P.n_workers)), dim3(kThreads), 0, stream, P);
  if (hipGetLastError() != hipSuccess) return SV_EHIP;
  return SV_OK;
}

int run(int dtype, const void* target, const void* draft, const int32_t* tokens,
        const int32_t* lens, const float* uniforms, int B, int D, int V, const float* temperature,
        int32_t* out_len, int32_t* out_tokens, void* ws, size_t ws_bytes, float* dbg_stats,
        int32_t* dbg_argmax, float* dbg_logpq, hipStream_t stream) {
  if (dtype != 0 && dtype != 1) return SV_EDTYPE;
  int rc = check_args(target, draft, tokens, uniforms, temperature, out_len, out_tokens, B, D, V);
  if (rc != SV_OK) return rc;
  Layout lay;
  make_layout(B, D, V, dtype == 1 ? 2 : 4, lay);
  const size_t need = workspace_bytes(B, D, V);
  if (ws != nullptr && (ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255)))
    return SV_ENOMEM;

  int dev = 0, count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return SV_ENODEV;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ENODEV;

  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if (ws == nullptr) {
    DeviceWorkspace& w = g_ws[{dev, stream}];
    if (w.bytes < need) {
      if (w.ptr) {
        // earlier calls on this stream may still use the old buffer
        if (hipStreamSynchronize(stream) != hipSuccess) return SV_EHIP;
        (void)hipFree(w.ptr);
        g_ws_state.erase(w.ptr);
        w.ptr = nullptr;
        w.bytes = 0;
      }
      if (hipMalloc(&w.ptr, need) != hipSuccess) { w.ptr = nullptr; return SV_ENOMEM; }
      if (hipMemset(w.ptr, 0, need) != hipSuccess) return SV_EHIP;   // counters start at zero
      w.bytes = need;
    }
    ws = w.ptr;
  }
  WsState& state = g_ws_state[ws];
  char* base = static_cast<char*>(ws);
  if (state.B >= 0 && (state.B != B || state.D != D)) {
    // the counter layout changed: clear both counter sets (a small kernel, graph-safe)
    const long long n = (long long)(2 * lay.set_bytes / 4);
    hipLaunchKernelGGL(clear_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<unsigned*>(base), n);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
  }
  state.B = B;
  state.D = D;
  const int parity = int(state.calls & 1);
  ++state.calls;

  Params P = {};
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
  P.R = 2 * D + 1;
  P.rch = lay.rch;
  P.nchunk = lay.nchunk;
  P.cur = counter_set(base, lay, parity);
  P.nxt = counter_set(base, lay, 1 - parity);
  P.rpart = reinterpret_cast<RowPart*>(base + lay.off_rpart);
  P.pinfo = reinterpret_cast<PosInfo*>(base + lay.off_pinfo);
  P.desc = reinterpret_cast<SeqDesc*>(base + lay.off_desc);
  P.fpart = reinterpret_cast<FinPart*>(base + lay.off_fpart);
  P.fmass = reinterpret_cast<double*>(base + lay.off_fmass);
  P.dbg_row_stats = dbg_stats;
  P.dbg_argmax = dbg_argmax;
  P.dbg_logpq = dbg_logpq;
  if (dbg_stats && hipMemsetAsync(dbg_stats, 0xff, size_t(B) * P.R * 2 * 4, stream) != hipSuccess)
    return SV_EHIP;                    // 0xffffffff: NaN for rows that are never evaluated
  if (dbg_argmax && hipMemsetAsync(dbg_argmax, 0xff, size_t(B) * (D + 1) * 4, stream) != hipSuccess)
    return SV_EHIP;                    // -1
  if (dbg_logpq && D > 0 && hipMemsetAsync(dbg_logpq, 0xff, size_t(B) * D * 2 * 4, stream) != hipSuccess)
    return SV_EHIP;
  return dtype == 1 ? launch<uint16_t>(P, dev, stream) : launch<float>(P, dev, stream);
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

size_t spec_verify_workspace_bytes(int B, int D, int V) { return sv::workspace_bytes(B, D, V); }

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

int spec_verify_version(void) { return 300; }

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
