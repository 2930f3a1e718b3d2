// Speculative-decoding verification sampler for MI355X (gfx950): kernels and C ABI.
//
// The operation is the one stated in include/spec_verify.h: accept / reject / residual rule
// from "Speculative Speculative Decoding - асинхронизируй это" (recap of standard speculative
// decoding), the bonus token from "Accélérer Sonar par la Spéculation" (section "Décodage
// spéculatif"), in-order acceptance up to the first mismatch and AL in [1, 1 + D] from
// "NVIDIA: öt irányelv ..." (section "Mit csinál a spekulatív dekódolás?").
//
// Kernels per call, in stream order: the row kernel (once, or in stages over the positions
// with a decision kernel between stages, so that rows past a rejection already known are not
// read), then (item grids of more than one round of resident workgroups only) the outcome
// kernel, the item kernel, and (then too) the pick kernel. Each hands its results to the next
// through the kernel boundary; no workgroup waits for another. Inside the item kernel, when its
// grid is one round, the workgroups of a sequence count their finished items (one atomic per
// workgroup) and the last one picks.
// Threshold acceptance runs the same kernels without the draft rows; the epilogue that moves
// each sequence's token window by AL is a kernel of its own, enqueued after verification.
//
// * Row kernel: one workgroup per 32 KB chunk of a row, position-major order (the position-0
//   target rows of the batch, then its position-0 draft rows, then position 1, ...). It streams
//   its chunk with non-temporal 16-byte loads and stores the chunk's exact max and fp32
//   sum exp((x - max) / T) (sampled rows) or max and lowest argmax (greedy target rows); the
//   chunk holding the draft token x_p also records the logit at x_p. Rows the method does not need (padding, draft rows of greedy
//   sequences, rows of invalid sequences) are not read.
// * Item kernel: one wavefront per final-draw item (b, f). The wavefront first derives sequence
//   b's outcome from the row partials: per-row statistics by a fixed combine tree, the test
//   u_p < min(1, p_p(x_p)/q_p(x_p)) (or x_p == argmax for greedy) at every position, the first
//   rejection j. Every wavefront of the sequence computes the same bits; item 0's writes the
//   accepted tokens, AL and the final-draw descriptor. An item covers kItemElems consecutive
//   elements of the final row(s) (target and draft row j after a rejection at j, target row L
//   for the bonus draw). It forms fp64 normalising sums and the residual mass linearised around
//   the fp32 estimate rho~ of rho = S_t / S_d: elements whose x_t - x_d puts ln(e_t / e_d)
//   clearly above ln rho~ are certainly in the positive part of p - q and contribute
//   e_t / S_t - e_d / S_d, those clearly below contribute nothing, those inside the band are
//   summed apart with the range of their x_t - x_d (one value means one exact ratio class,
//   resolved exactly by the pick).
// * Pick: one wavefront per sequence. Exact normalisers from the item sums, the item masses,
//   the item and block holding u * Z, and an fp64 prefix-scan rescan of that block give the
//   token. When every item workgroup of the call is resident at once, the item workgroup that
//   completes a sequence's count picks (no third kernel); otherwise a pick kernel runs after
//   the item kernel.
// * Decision kernel (staged row launches only): one wavefront per sequence evaluates the
//   positions read so far exactly as the outcome does and stores the first that rejects; the
//   next row launch skips the rows past it. AL and the tokens do not depend on those rows, and
//   the outcome, which later reads every row partial up to L, takes the first rejection, so the
//   stale partials of skipped rows (all past it) never decide anything.
// * Outcome kernel: only when the item grid takes more than one round of resident workgroups
//   (large batches). One wavefront per sequence derives the outcome once, between the row and
//   item kernels, and the item workgroups read it with one load instead of deriving it each.
#include <hip/hip_ext.h>
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
constexpr int kFinBlock = 64 * kFinPer;       // elements per wavefront block (512)
constexpr int kItemsPerChunk = 8;             // final-draw items per row chunk length
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Half-width of the band (in ln(e_t/e_d)) inside which an element's sign in max(0, p - q) is
// not decided from the fp32 estimate of ln(S_t/S_d). The fp32 statistics are accurate to a
// few 1e-6, so the exact ln(S_t/S_d) lies well inside; the pick checks that it does.
constexpr double kBand = 3e-5;

// kind of a sequence's final token, in its outcome words
enum Mode : unsigned { kNoDraw = 1, kResidual = 2, kBonus = 3 };

struct RowPart {      // partial statistics of one row chunk
  float m;            // max of the raw logits in the chunk
  float s;            // sampled rows: sum exp((x - m) / T); greedy rows: bits of the argmax
  float xv;           // logit at the draft token of this position, if it lies in the chunk
  float pad;
};

// Outcome of one sequence as handed to the pick kernel: two 64-bit words.
struct SeqPub {
  unsigned long long a;   // bits 0-1 Mode, 2-6 position j of the final draw, 32-63 bits of
                          // the exact max of target row j
  unsigned long long c;   // bits 0-31 bits of the exact max of draft row j, 32-63 bits of the
                          // fp32 ln(S_t / S_d) of row j with its lowest bit forced to 1 (a
                          // marker that a draw is due; moves the estimate by one ulp, far
                          // inside the band)
};

constexpr int kMaxItemBlocks = 4;

struct FinPart {      // fp64 sums of one final-draw item
  double st, sd;      // sum e_t, sum e_d   (e = exp((x - max) / T))
  double at, ad;      // sums over elements certainly in the positive part of p - q
  double bt, bd;      // sums over the elements inside the band
  double dmin, dmax;  // min / max of x_t - x_d inside the band (+inf / -inf: none)
  double kat[kMaxItemBlocks], kad[kMaxItemBlocks];   // at, ad of each 512-element block
                                                     // (bonus draws: kat = e_t per block)
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
  int b0, nb;         // the sequences [b0, b0 + nb) of this launch (grid y covers nb or 2 nb)
  int R;              // rows per sequence, 2D + 1 (target 0..D, then draft 0..D-1)
  int rch;            // elements per row chunk
  int nchunk;         // row chunks per row
  int fch;            // elements per final-draw item (rch / kItemsPerChunk, a multiple of 512)
  int nF;             // final-draw items per sequence
  SeqPub* pub;        // [B] outcome of each sequence (item kernel -> pick kernel)
  RowPart* rpart;     // [B][R][nchunk]
  FinPart* fpart;     // [B][nF]
  double* fmass;      // [B][nF] scratch of the pick
  unsigned* done;     // [B] item workgroups finished (when the last one picks)
  int p_lo;           // first position of this row launch (its grid z covers p_lo ..)
  const unsigned* dead;  // [B] or null: the first position already known to reject (rows past
                         // it are not read); 0xffffffff when none is known
  unsigned* dead_buf;    // [B] where the decision kernel stores it
  int merged;         // 1: the last item workgroup of a sequence does its pick
  int pre;            // 1: the outcome kernel has stored every outcome (item grids of more
                      //    than one round); item workgroups read it instead of deriving it
  int stage;          // 1: staged row launches that skip the rows past a known rejection
  int thresh;         // 1: threshold acceptance (prefix probability above tau; no draft rows)
  double log_tau;     // ln tau of threshold acceptance (-inf for tau = 0)
  float* dbg_row_stats;  // optional [B][R][2]
  int32_t* dbg_argmax;   // optional [B][D+1]
  float* dbg_logpq;      // optional [B][D][2]
};

// ------------------------------------------------------------------------------------------
// device-coherent accesses (item records that a pick in the same kernel may read; the pick's
// scratch masses: one lane stores, others load them back)

template <typename T>
__device__ inline void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ inline T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A load that is device-coherent when COH (data another workgroup of the same kernel stored with
// st_dev), a plain one otherwise (data of an earlier kernel).
template <bool COH, typename T>
__device__ inline T ld_rec(const T* p) {
  if constexpr (COH) return ld_dev(p);
  else return *p;
}

__device__ inline unsigned add_dev(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wavefront's earlier vector-memory operations (the stores of the scratch
// masses) have completed, before they are loaded back.
__device__ inline void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------------------------------------
// element access

// A load from global memory through a generic pointer (a global, not a flat, access).
template <typename T>
__device__ inline T ld_global(const T* p) {
  return *(__attribute__((address_space(1))) const T*)p;
}

template <typename E> struct Elem;
// Running maximum of packed values. bf16 pairs are compared as fp16 pairs (one packed max per
// word): both formats are sign-magnitude with the magnitude ordered like its bit pattern, so
// the fp16 order of the halves is the bf16 order of the values they hold, for every bf16 value
// below 2^121 in magnitude. The larger ones fall on fp16's inf / NaN patterns, which the packed
// max passes over (quiet NaN), returns (inf) or turns into the canonical NaN (signalling NaN);
// the row chunk detects each outcome and redoes its max exactly.
__device__ inline uint32_t pk_max_bf16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <> struct Elem<uint16_t> {          // bf16 bit patterns
  static constexpr int kVec = 8;             // elements per 16-byte load
  __device__ static float get(const uint16_t* p, size_t i) {
    return __uint_as_float(uint32_t(ld_global(p + i)) << 16);
  }
  __device__ static float lane(const uint4& v, int e) {
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  static constexpr uint32_t kNegInf = 0xff80ff80u;    // two bf16 -inf (fp16 quiet NaNs: a
                                                       // packed max passes them over)
  // packed running max (see pk_max_bf16); identity: the packed pattern of two -inf (fp16)
  typedef uint32_t Acc;
  __device__ static Acc acc_init() { return 0xfc00fc00u; }
  __device__ static Acc acc_add(Acc a, const uint4& v) {
    return pk_max_bf16(pk_max_bf16(a, v.x), pk_max_bf16(pk_max_bf16(v.y, v.z), v.w));
  }
  __device__ static float acc_value(Acc a) {
    return fmaxf(__uint_as_float(a << 16), __uint_as_float(a & 0xffff0000u));
  }
};
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float get(const float* p, size_t i) { return ld_global(p + i); }
  __device__ static float lane(const uint4& v, int e) {
    return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
  }
  static constexpr uint32_t kNegInf = 0xff800000u;
  typedef float Acc;
  __device__ static Acc acc_init() { return -INFINITY; }
  __device__ static Acc acc_add(Acc a, const uint4& v) {
    return fmaxf(fmaxf(a, __uint_as_float(v.x)),
                 fmaxf(fmaxf(__uint_as_float(v.y), __uint_as_float(v.z)), __uint_as_float(v.w)));
  }
  __device__ static float acc_value(Acc a) { return a; }
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 global_u32x4;

// Non-temporal 16-byte load. The logits are global memory; saying so makes it a global (not a
// flat) load, which counts against the vector-memory counter only.
__device__ inline uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load((global_u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The run p[a .. a+n), n <= kFinPer, zero past n, kept packed as loaded (16-byte loads when
// aligned; element loads otherwise, packed the same way).
template <typename E> struct Run;
template <> struct Run<uint16_t> {
  uint32_t w[4];
  __device__ __forceinline__ void load(const uint16_t* p, int a, int n) {
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
  // the full run at q, 16-byte aligned
  __device__ __forceinline__ void load_vec(const uint16_t* q) {
    const uint4 v = *reinterpret_cast<const uint4*>(q);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
  __device__ float at(int e) const {
    return __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
  }
};
template <> struct Run<float> {
  float x[kFinPer];
  __device__ __forceinline__ void load(const float* p, int a, int n) {
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
  __device__ __forceinline__ void load_vec(const float* q) {
    const float4 v0 = reinterpret_cast<const float4*>(q)[0];
    const float4 v1 = reinterpret_cast<const float4*>(q)[1];
    x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
    x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
  }
  __device__ float at(int e) const { return x[e]; }
};

// wave-uniform values kept in scalar registers
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ inline bool seq_valid(int L, int D, float T) {
  return L >= 0 && L <= D && isfinite(T) && T >= 0.f;
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

// Reduction of a float over the wavefront with DPP row shifts and row broadcasts (the steps of
// dpp_scan below), the total read from lane 63 into every lane. Needs every lane active.
template <int CTRL, int ROWS>
__device__ inline float dpp_float(float x, float id) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(x), CTRL,
                                                    ROWS, 0xf, false));
}
template <typename Op>
__device__ inline float dpp_total(float x, float id, Op op) {
  x = op(x, dpp_float<0x111, 0xf>(x, id));   // row_shr:1
  x = op(x, dpp_float<0x112, 0xf>(x, id));   // row_shr:2
  x = op(x, dpp_float<0x114, 0xf>(x, id));   // row_shr:4
  x = op(x, dpp_float<0x118, 0xf>(x, id));   // row_shr:8
  x = op(x, dpp_float<0x142, 0xa>(x, id));   // row_bcast:15
  x = op(x, dpp_float<0x143, 0xc>(x, id));   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// (max, sum exp2((x - max) k)) over the wavefront: the max first, then each lane's sum rescaled
// to it and added up (one exp2 per lane). Every lane gets the result.
__device__ inline void wave_ms(float& m, float& s, float k) {
  const float mw = dpp_total(m, -INFINITY, [](float a, float b) { return fmaxf(a, b); });
  const float sr = (s == 0.f) ? 0.f : s * __builtin_amdgcn_exp2f((m - mw) * k);
  s = dpp_total(sr, 0.f, [](float a, float b) { return a + b; });
  m = mw;
}

// Argmax over the wavefront with the DPP steps of dpp_total (am_combine is associative and
// commutative); every lane gets lane 63's result. Needs every lane active.
template <int CTRL, int ROWS>
__device__ inline void am_step(float& v, int& i) {
  const float v2 = dpp_float<CTRL, ROWS>(v, -INFINITY);
  const int i2 = __builtin_amdgcn_update_dpp(-1, i, CTRL, ROWS, 0xf, false);
  am_combine(v, i, v2, i2);
}
__device__ inline void wave_am(float& v, int& i) {
  am_step<0x111, 0xf>(v, i);
  am_step<0x112, 0xf>(v, i);
  am_step<0x114, 0xf>(v, i);
  am_step<0x118, 0xf>(v, i);
  am_step<0x142, 0xa>(v, i);
  am_step<0x143, 0xc>(v, i);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

// Natural log and exp from the hardware base-2 instructions (relative error near 1e-7; the
// accept tests and the band around ln(S_t / S_d) need 1e-5).
__device__ inline float ln_hw(float x) { return __builtin_amdgcn_logf(x) * kLn2; }
__device__ inline float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// ms_combine without branches, for operands that are either empty (m = -inf, s = 0) or
// non-empty (s > 0); the same result for (a, b) as for (b, a).
__device__ inline void ms_merge(float& m, float& s, float m2, float s2, float k) {
  const float mn = fmaxf(m, m2);
  const float a = s == 0.f ? 0.f : s * __builtin_amdgcn_exp2f((m - mn) * k);
  const float c = s2 == 0.f ? 0.f : s2 * __builtin_amdgcn_exp2f((m2 - mn) * k);
  s = a + c;
  m = mn;
}

// Inclusive scans of a double over the 64 lanes with DPP row shifts and row broadcasts (VALU
// only, no LDS traffic): Hillis-Steele within rows of 16, then row 0's total into row 1 and
// row 2's into row 3, then the total of rows 0-1 into rows 2 and 3. Lane 63 ends with the
// reduction of all lanes. Lanes a shift reads from outside the row contribute `id` (the
// operation's identity).
template <int CTRL, int ROWS>
__device__ inline double dpp_double(double x, double id) {
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(id), __double2loint(x), CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(id), __double2hiint(x), CTRL, ROWS, 0xf, false);
  return __hiloint2double(hi, lo);
}
template <typename Op>
__device__ inline double dpp_scan(double x, double id, Op op) {
  x = op(x, dpp_double<0x111, 0xf>(x, id));   // row_shr:1
  x = op(x, dpp_double<0x112, 0xf>(x, id));   // row_shr:2
  x = op(x, dpp_double<0x114, 0xf>(x, id));   // row_shr:4
  x = op(x, dpp_double<0x118, 0xf>(x, id));   // row_shr:8
  x = op(x, dpp_double<0x142, 0xa>(x, id));   // row_bcast:15 into rows 1 and 3
  x = op(x, dpp_double<0x143, 0xc>(x, id));   // row_bcast:31 into rows 2 and 3
  return x;
}

// The sum scan: the row shifts read 0 from outside the row (bound_ctrl) instead of an identity
// moved into the destination first; the same additions in the same order as dpp_scan.
template <int CTRL>
__device__ inline double dpp_shr_zero(double x) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), CTRL, 0xf, 0xf, true);
  return __hiloint2double(hi, lo);
}
__device__ inline double dpp_scan_add(double x) {
  x += dpp_shr_zero<0x111>(x);                // row_shr:1
  x += dpp_shr_zero<0x112>(x);                // row_shr:2
  x += dpp_shr_zero<0x114>(x);                // row_shr:4
  x += dpp_shr_zero<0x118>(x);                // row_shr:8
  x += dpp_double<0x142, 0xa>(x, 0.0);        // row_bcast:15 into rows 1 and 3
  x += dpp_double<0x143, 0xc>(x, 0.0);        // row_bcast:31 into rows 2 and 3
  return x;
}
// value of lane l (wave-uniform l)
__device__ inline double readlane(double x, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), l),
                          __builtin_amdgcn_readlane(__double2loint(x), l));
}
// sum over the wavefront, in every lane
__device__ inline double wave_total(double x) { return readlane(dpp_scan_add(x), 63); }
// lane i gets lane i - 1's x, lane 0 gets first
__device__ inline double lane_before(double x, double first) {
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(first), __double2loint(x), 0x138, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(first), __double2hiint(x), 0x138, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

__device__ inline double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// ------------------------------------------------------------------------------------------
// shared memory of one workgroup

struct Shared {
  float red[kWaves][2];         // cross-wavefront combine of the row chunk
};

// ------------------------------------------------------------------------------------------
// row chunk: statistics of one 32 KB chunk (whole workgroup), stored by wavefront 0

template <typename E>
__device__ __forceinline__ void row_chunk(const Params& P, Shared& sm, int b, int p, int which,
                                          int c, int L, float T, bool greedy, int tid) {
  constexpr int kV = Elem<E>::kVec;
  const int D = P.D, nc = P.nchunk;
  const int r = which == 0 ? p : D + 1 + p;
  const E* row = which == 0
      ? static_cast<const E*>(P.target) + (size_t(b) * (D + 1) + p) * size_t(P.V)
      : static_cast<const E*>(P.draft) + (size_t(b) * D + p) * size_t(P.V);
  const int c0 = c * P.rch;
  const int n = min(P.rch, P.V - c0);
  const E* ptr = row + c0;
  const bool aligned = (reinterpret_cast<uintptr_t>(ptr) & 15) == 0;
  const int nvec = aligned ? n / kV : 0;

  // the thread's vectors tid + 256 k; past nvec they hold -inf (no weight, never the max), and
  // the load repeats the last vector so that every load is unconditional
  const uint4* vp = reinterpret_cast<const uint4*>(ptr);
  uint4 buf[kRowVecs];
  if (nvec == kRowVecs * kThreads) {
#pragma unroll
    for (int k = 0; k < kRowVecs; ++k) buf[k] = load_stream(vp + tid + k * kThreads);
  } else {
    const uint4 ninf = make_uint4(Elem<E>::kNegInf, Elem<E>::kNegInf, Elem<E>::kNegInf,
                                  Elem<E>::kNegInf);
#pragma unroll
    for (int k = 0; k < kRowVecs; ++k) {
      const int vi = tid + k * kThreads;
      buf[k] = ninf;
      if (nvec > 0) {
        const uint4 v = load_stream(vp + min(vi, nvec - 1));
        if (vi < nvec) buf[k] = v;
      }
    }
  }
  float xv = 0.f;
  if (!greedy && tid == 0 && p < L) {
    const int x = P.tokens[size_t(b) * D + p];
    if (x >= c0 && x < c0 + n) xv = Elem<E>::get(row, x);
  }

  const int wave = tid >> 6;
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
    if ((tid & 63) == 0) { sm.red[wave][0] = best; sm.red[wave][1] = __int_as_float(bi); }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 1; w < kWaves; ++w) am_combine(best, bi, sm.red[w][0], __float_as_int(sm.red[w][1]));
    m = best;
    s = __int_as_float(bi < 0 ? -1 : c0 + bi);
  } else {
    // the thread's max over its vectors (packed), then one pass of exp2 sums against it
    const float k2 = kLog2e / T;
    typename Elem<E>::Acc acc = Elem<E>::acc_init();
#pragma unroll
    for (int k = 0; k < kRowVecs; ++k) acc = Elem<E>::acc_add(acc, buf[k]);
    float mx = tid < nvec ? Elem<E>::acc_value(acc) : -INFINITY;
    float sum = 0.f;
    if (tid < nvec) {
      const float off = -mx * k2;
#pragma unroll
      for (int k = 0; k < kRowVecs; ++k) {
#pragma unroll
        for (int e = 0; e < kV; ++e)
          sum += __builtin_amdgcn_exp2f(fmaf(Elem<E>::lane(buf[k], e), k2, off));
      }
    }
    // Exact redo where the packed max may not be the max: it landed on an fp16 inf / NaN
    // pattern (|value| >= 2^121, or a thread whose elements are all -inf), or passed over such a
    // value and the sum overflowed or became NaN (-inf - -inf). -inf elements (masked tokens)
    // carry no weight.
    if (!(sum < INFINITY) || !(fabsf(mx) < 0x1p121f)) {
      mx = -INFINITY;
      sum = 0.f;
      for (int k = 0; k < kRowVecs; ++k) {
        if (tid + k * kThreads < nvec) {
          for (int e = 0; e < kV; ++e) {
            const float x = Elem<E>::lane(buf[k], e);
            if (x > mx) {
              sum = (sum == 0.f) ? 0.f : sum * __builtin_amdgcn_exp2f((mx - x) * k2);
              mx = x;
            }
            if (x > -INFINITY) sum += __builtin_amdgcn_exp2f((x - mx) * k2);
          }
        }
      }
    }
    for (int i = nvec * kV + tid; i < n; i += kThreads) {
      const float x = Elem<E>::get(ptr, i);
      if (x > mx) {
        sum = (sum == 0.f) ? 0.f : sum * __builtin_amdgcn_exp2f((mx - x) * k2);
        mx = x;
      }
      if (x > -INFINITY) sum += __builtin_amdgcn_exp2f((x - mx) * k2);
    }
    wave_ms(mx, sum, k2);
    if ((tid & 63) == 0) { sm.red[wave][0] = mx; sm.red[wave][1] = sum; }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 1; w < kWaves; ++w) ms_combine(mx, sum, sm.red[w][0], sm.red[w][1], k2);
    m = mx;
    s = sum;
  }

  if (tid == 0) {
    RowPart* out = P.rpart + (size_t(b) * P.R + r) * nc + c;
    *out = RowPart{m, s, xv, 0.f};
  }
}

// ------------------------------------------------------------------------------------------
// outcome of a sequence, from its row partials (one wavefront)

struct Outcome {
  unsigned mode;      // kNoDraw (greedy or invalid row), kResidual or kBonus
  int j;              // position of the final token
  float mt, md;       // exact maxima of target row j and (residual) draft row j
  float lnrho;        // residual: fp32 ln(S_t / S_d) of row j, lowest bit forced to 1
  float u;            // the final draw's uniform
};

constexpr int kPartBatch = 8;   // chunk partials a lane loads at once

// The statistics of row r (lane r) from chunk partials c0 .. c0 + 7 (those below nc), merged
// into (m, s, x): max first, then one exp2 per chunk.
__device__ inline void merge_batch(const RowPart (&q)[kPartBatch], int c0, int nc, float k2,
                                   float& m, float& s, float& x) {
  float mb = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPartBatch; ++i)
    if (c0 + i < nc) mb = fmaxf(mb, q[i].m);
  float sb = 0.f;
#pragma unroll
  for (int i = 0; i < kPartBatch; ++i)
    if (c0 + i < nc && q[i].s != 0.f) sb = fmaf(q[i].s, __builtin_amdgcn_exp2f((q[i].m - mb) * k2), sb);
#pragma unroll
  for (int i = 0; i < kPartBatch; ++i)
    if (c0 + i < nc) x += q[i].xv;     // zero except in the chunk holding the draft token
  ms_merge(m, s, mb, sb, k2);
}
__device__ inline void argmax_batch(const RowPart (&q)[kPartBatch], int c0, int nc, float& v,
                                    int& idx) {
#pragma unroll
  for (int i = 0; i < kPartBatch; ++i)
    if (c0 + i < nc) am_combine(v, idx, q[i].m, __float_as_int(q[i].s));
}

// What the outcome of a sequence reads, loaded in one go: lane r < R the first batch of row r's
// chunk partials (target rows 0..D, then draft rows 0..D-1; loaded whether the row is needed or
// not, the workspace being always readable), lane p its draft token and uniform.
struct OutcomeIn {
  RowPart q[kPartBatch];
  int L;
  float T;
  int xl;
  float ul;
};

__device__ __forceinline__ OutcomeIn load_outcome(const Params& P, int b, int lane) {
  const int D = P.D, R = P.R, nc = P.nchunk;
  OutcomeIn in;
  const RowPart* rp = P.rpart + (size_t(b) * R + lane) * nc;
#pragma unroll
  for (int i = 0; i < kPartBatch; ++i)
    if (lane < R && i < nc) in.q[i] = rp[i];
  in.L = P.lens ? P.lens[b] : D;
  in.T = P.temperature[b];
  in.xl = lane < D ? P.tokens[size_t(b) * D + lane] : 0;
  in.ul = lane <= D ? P.uniforms[size_t(b) * (D + 1) + lane] : 0.f;
  return in;
}

// Every wavefront that computes the outcome of sequence b from the same partials gets the same
// bits (fixed combine order). With `write`, the wavefront also stores AL, the tokens other than
// the final draw's, the outcome words and the debug exports.
// limit: only positions below it are evaluated (their rows merged); the outcome is then valid
// for them only (the decision kernel between staged row launches).
template <typename E>
__device__ __forceinline__ Outcome seq_outcome(const Params& P, int b, const OutcomeIn& in,
                                               int lane, bool write, int limit = 64) {
  const int D = P.D, R = P.R, nc = P.nchunk;
  // Lane r < R holds row r and combines its chunk partials in order.
  const int r = lane;
  const RowPart* rp = P.rpart + (size_t(b) * R + r) * nc;
  RowPart q[kPartBatch];
#pragma unroll
  for (int i = 0; i < kPartBatch; ++i) q[i] = in.q[i];
  const int L = in.L;
  const float T = in.T;
  const int xl = in.xl;
  const float ul = in.ul;
  int32_t* toks = P.out_tokens + size_t(b) * (D + 1);

  Outcome o = {kNoDraw, 0, 0.f, 0.f, 0.f, 0.f};
  bool valid = seq_valid(L, D, T);
  if (valid) valid = !__any(lane < L && (xl < 0 || xl >= P.V));    // L <= D <= 31
  if (!valid) {                        // the row is marked: AL 0, tokens -1
    if (write) {
      for (int i = lane; i <= D; i += 64) toks[i] = -1;
      if (lane == 0) {
        P.out_len[b] = 0;
        P.pub[b] = SeqPub{(unsigned long long)kNoDraw, 0ull};
      }
    }
    return o;
  }
  const bool greedy = (T == 0.f);
  const float iT = 1.f / T;
  const float k2 = kLog2e * iT;
  const int pr = r <= D ? r : r - (D + 1);
  const bool need = r < R && pr < limit &&
                    (r <= D ? pr <= L : (!greedy && !P.thresh && pr < L));
  float m = -INFINITY, s = 0.f, x = 0.f;
  int idx = -1;
  if (need) {
    if (greedy) argmax_batch(q, 0, nc, m, idx);
    else merge_batch(q, 0, nc, k2, m, s, x);
    for (int c0 = kPartBatch; c0 < nc; c0 += kPartBatch) {
#pragma unroll
      for (int i = 0; i < kPartBatch; ++i)
        if (c0 + i < nc) q[i] = rp[c0 + i];
      if (greedy) argmax_batch(q, c0, nc, m, idx);
      else merge_batch(q, c0, nc, k2, m, s, x);
    }
  }
  // position p = lane: target row p is this lane's, draft row p is lane D + 1 + p's
  const int dl = min(D + 1 + lane, 63);
  const float md_l = __shfl(m, dl), sd_l = __shfl(s, dl), xd_l = __shfl(x, dl);
  // position p = lane: its test
  const int p = lane;
  bool rej = false;
  int g = -1;
  float mt = 0.f, md = 0.f, lr = 0.f, lpx = 0.f;
  if (p <= L) {
    if (greedy) {
      g = idx;
      if (p < L) rej = xl != g;
      if (write && P.dbg_argmax) P.dbg_argmax[size_t(b) * (D + 1) + p] = g;
    } else {
      mt = m;
      const float lnt = ln_hw(s);
      float lnd = 0.f;
      if (p < L && P.thresh) {
        lpx = (x - mt) * iT - lnt;     // the test is taken below, on the running sum
        if (write && P.dbg_logpq) {
          P.dbg_logpq[(size_t(b) * D + p) * 2] = lpx;
          P.dbg_logpq[(size_t(b) * D + p) * 2 + 1] = __int_as_float(0x7fc00000);
        }
      } else if (p < L) {
        md = md_l;
        lnd = ln_hw(sd_l);
        const float lp = (x - mt) * iT - lnt;
        const float lq = (xd_l - md) * iT - lnd;
        const float ratio = exp_hw(lp - lq);
        rej = !(ul < fminf(1.f, ratio));
        lr = __uint_as_float(__float_as_uint(lnt - lnd) | 1u);
        if (write && P.dbg_logpq) {
          P.dbg_logpq[(size_t(b) * D + p) * 2] = lp;
          P.dbg_logpq[(size_t(b) * D + p) * 2 + 1] = lq;
        }
        if (write && P.dbg_row_stats) {
          P.dbg_row_stats[(size_t(b) * R + D + 1 + p) * 2] = md / T;
          P.dbg_row_stats[(size_t(b) * R + D + 1 + p) * 2 + 1] = lnd;
        }
      }
      if (write && P.dbg_row_stats) {
        P.dbg_row_stats[(size_t(b) * R + p) * 2] = mt / T;
        P.dbg_row_stats[(size_t(b) * R + p) * 2 + 1] = lnt;
      }
    }
  }
  if (P.thresh && !greedy) {
    // threshold acceptance ("Accélérer Sonar par la Spéculation", "Décodage spéculatif"): the
    // prefix through position p is kept while sum_{i<=p} log p_i(x_i) > ln tau; the running sum
    // in fp64 over the fp32 log-probabilities, lane p holding position p
    const double cs = dpp_scan_add(p < L ? double(lpx) : 0.0);
    rej = p < L && !(cs > P.log_tau);
  }
  const unsigned long long rejm = __ballot(rej);
  const int j = rejm ? int(__builtin_ctzll(rejm)) : L;
  o.j = j;
  // threshold acceptance draws the extra token from p_j at a rejection too (no residual)
  o.mode = greedy ? kNoDraw : ((j < L && !P.thresh) ? kResidual : kBonus);
  o.mt = __shfl(mt, j);
  o.md = __shfl(md, j);
  o.lnrho = __shfl(lr, j);
  o.u = __shfl(ul, D);
  if (write) {
    if (lane <= D) {
      if (greedy) toks[lane] = lane <= j ? g : -1;
      else if (lane < j) toks[lane] = xl;
      else if (lane > j) toks[lane] = -1;      // position j is written by the final draw
    }
    if (lane == 0) {
      P.out_len[b] = j + 1;
      const unsigned long long a = greedy ? (unsigned long long)kNoDraw
          : ((unsigned long long)__float_as_uint(o.mt) << 32) | (o.mode | (unsigned(j) << 2));
      const unsigned long long c = greedy ? 0ull
          : ((unsigned long long)(__float_as_uint(o.lnrho) | 1u) << 32) | __float_as_uint(o.md);
      P.pub[b] = SeqPub{a, c};
    }
  }
  return o;
}

// ------------------------------------------------------------------------------------------
// final draw
//
// A final-draw item covers kItemElems<E> consecutive elements of the final row(s) of one
// sequence (2048 bf16 or 1024 fp32 logits), in blocks of 512: lane l handles elements
// 512k + 8l .. 512k + 8l + 7 of block k, and loads all of them at once. One wavefront per item.
//
// Weights are e(x) = exp((x - m) / T) in fp64 (m the row's exact max). Exponents are carried in
// units of ln2/256: y = (x - m) / T * 256 / ln 2 = fma(x, c1, c0) with c1 = 256 / (T ln 2) and
// c0 = -m c1, so that e = 2^(y / 256); for |x - m| / T up to 30 the rounding of c1, c0 and of
// the fma moves y by a few 1e-12, i.e. e by a few 1e-15 relative.

template <typename E>
constexpr int kItemElems = kRowChunkBytes / int(sizeof(E)) / kItemsPerChunk;
template <typename E>
constexpr int kItemBlocks = kItemElems<E> / kFinBlock;
static_assert(kItemBlocks<uint16_t> <= kMaxItemBlocks && kItemBlocks<float> <= kMaxItemBlocks,
              "an item record holds the masses of at most kMaxItemBlocks blocks");

// 2^(y / 256) = 2^(k / 256) * 2^(r / 256), k = rint(y), r = y - k in [-1/2, 1/2] (exact);
// 1 / k!, k = 0..17 (k! is exact in a double up to 17!)
struct InvFactorials {
  double v[18];
  constexpr InvFactorials() : v() {
    double f = 1.0;
    v[0] = 1.0;
    for (int k = 1; k < 18; ++k) {
      f *= k;
      v[k] = 1.0 / f;
    }
  }
};
constexpr InvFactorials kInvFact;

// The table e2[i] = 2^(i / 256), i = 0..255, in shared memory: e^x at x = i ln2 / 256 <= 0.7 from
// its Taylor polynomial of degree 17 (truncation below 3e-18 relative), Horner form.
__device__ inline void fill_e2(double* e2, int tid) {
  constexpr double c = 0.0027076061740622863;          // ln2 / 256
  for (int i = tid; i < 256; i += kThreads) {
    const double x = double(i) * c;
    double p = kInvFact.v[17];
#pragma unroll
    for (int k = 16; k >= 0; --k) p = fma(p, x, kInvFact.v[k]);
    e2[i] = p;
  }
}

// 2^(r / 256) = e^u with u = r ln2 / 256, |u| <= a = ln2 / 512, from a cubic: the Taylor cubic
// with the u^4 term economised by the Chebyshev polynomial T4 (u^4 ~ a^2 u^2 - a^4 / 8, off by
// at most a^4 / 8), relative error below 2e-14; 2^(k / 256) = e2[k mod 256] * 2^(k div 256).
// The argument is first raised to at least -2^30, so that a -inf logit (a masked token), or any
// argument far below zero, keeps k in int range and gives 0 through ldexp's underflow.
// k = rint(y) comes from adding 1.5 * 2^52: the sum's low 32 bits hold k (two's complement, for
// |y| < 2^31) and subtracting the constant again gives kf exactly, with no conversion
// instruction.
__device__ inline double exp2k(double y, const double* e2) {
  constexpr double c = 0.0027076061740622863;          // ln2 / 256
  constexpr double a2 = c * c / 4;                     // a^2
  constexpr double q0 = 1.0 - a2 * a2 / 192, q1 = c, q2 = (0.5 + a2 / 24) * c * c,
                   q3 = c * c * c / 6;
  constexpr double kRound = 6755399441055744.0;       // 1.5 * 2^52
  y = fmax(y, -0x1p30);
  const double t = y + kRound;
  const double kf = t - kRound;
  const double r = y - kf;
  const int k = int(uint32_t(__double_as_longlong(t)));
  const double p = fma(fma(fma(r, q3, q2), r, q1), r, q0);
  return ldexp(e2[k & 255] * p, k >> 8);
}

// e(x) of one final row.
struct RowExp {
  double c1, c0;        // y = fma(x, c1, c0)
  const double* e2;     // 2^(i/256), shared memory
  __device__ double operator()(float x) const { return exp2k(fma(double(x), c1, c0), e2); }
};

struct Draw {           // what the fp64 evaluation of one sequence's final row(s) needs
  bool residual;
  int j;
  RowExp t, d;          // target row j, draft row j
  double dhi, dlo;      // band of x_t - x_d: T (ln(rho~) +/- kBand) + m_t - m_d
  double lnrho, u;
};

// The draw of sequence b from its outcome (wave-uniform); e2 in shared memory.
__device__ inline Draw make_draw(const Params& P, int b, const Outcome& o, const double* e2) {
  constexpr double k256 = 369.3299304675746;          // 256 / ln 2
  Draw w;
  w.residual = o.mode == kResidual;
  w.j = o.j;
  const double T = double(P.temperature[b]);
  w.u = double(o.u);
  w.lnrho = double(o.lnrho);
  const double mt = double(o.mt);
  const double md = double(o.md);
  const double c1 = k256 / T;
  w.t = RowExp{c1, -mt * c1, e2};
  w.d = RowExp{c1, -md * c1, e2};
  w.dhi = T * (w.lnrho + kBand) + (mt - md);
  w.dlo = T * (w.lnrho - kBand) + (mt - md);
  return w;
}

template <typename E>
__device__ inline const E* final_row(const Params& P, int b, int j, bool draft) {
  return draft ? static_cast<const E*>(P.draft) + (size_t(b) * P.D + j) * size_t(P.V)
               : static_cast<const E*>(P.target) + (size_t(b) * (P.D + 1) + j) * size_t(P.V);
}

// One lane's elements of one item: block k holds elements a0 + 512k + 8 lane + (0..7).
template <typename E>
struct ItemRuns {
  Run<E> r[kItemBlocks<E>];
  __device__ __forceinline__ void load(const E* row, int a0, int V, int lane) {
#pragma unroll
    for (int k = 0; k < kItemBlocks<E>; ++k) {
      const int a = a0 + kFinBlock * k + kFinPer * lane;
      const int n = max(0, min(kFinPer, V - a));
      if (n > 0) r[k].load(row, a, n);
    }
  }
};

// Target runs, and draft runs when `both`, block by block (block 0's pair arrives first).
template <typename E>
__device__ __forceinline__ void load_item(ItemRuns<E>& t, ItemRuns<E>& d, const E* trow,
                                          const E* drow, bool both, int a0, int V, int lane) {
#pragma unroll
  for (int k = 0; k < kItemBlocks<E>; ++k) {
    const int a = a0 + kFinBlock * k + kFinPer * lane;
    const int n = max(0, min(kFinPer, V - a));
    if (n > 0) {
      t.r[k].load(trow, a, n);
      if (both) d.r[k].load(drow, a, n);
    }
  }
}

// Exact weight of element e of the runs: e_t when target_only, else max(0, e_t/S_t - e_d/S_d).
template <typename E>
__device__ inline double exact_weight(const Run<E>& rt, const Run<E>& rd, int e, const Draw& w,
                                      bool target_only, double it, double id) {
  const double et = w.t(rt.at(e));
  if (target_only) return et;
  const double ed = w.d(rd.at(e));
  return fmax(0.0, et * it - ed * id);
}

// Sum of the exact weights of one item's elements (fixed order); target_only as above. Only
// for the rare sequences whose band did not resolve every element.
template <typename E>
__device__ inline double item_exact_mass(const Params& P, const E* trow, const E* drow,
                                         const Draw& w, int f, bool target_only, double it,
                                         double id, int lane) {
  const int a0 = f * kItemElems<E>;
  ItemRuns<E> t, d;
  t.load(trow, a0, P.V, lane);
  if (!target_only) d.load(drow, a0, P.V, lane);
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kItemBlocks<E>; ++k) {
    const int n = max(0, min(kFinPer, P.V - (a0 + kFinBlock * k + kFinPer * lane)));
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) {
      if (e < n) s += exact_weight<E>(t.r[k], d.r[k], e, w, target_only, it, id);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  return wave_sum(s);
}

// The pick of a sequence: exact normalisers, item masses, token (one wavefront). Up to 64 items
// the item records are read once, one per lane (r); beyond, they are re-read per pass.
// The item records of sequence b that one pass of 64 lanes holds (all of them up to 64 items):
// lane l gets item l's.
template <bool COH>
__device__ inline FinPart first_records(const Params& P, int b, int lane) {
  FinPart r = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, INFINITY, -INFINITY};
  if (P.nF <= 64 && lane < P.nF) {
    const FinPart& q = P.fpart[size_t(b) * P.nF + lane];
    r.st = ld_rec<COH>(&q.st); r.sd = ld_rec<COH>(&q.sd);
    r.at = ld_rec<COH>(&q.at); r.ad = ld_rec<COH>(&q.ad);
    r.bt = ld_rec<COH>(&q.bt); r.bd = ld_rec<COH>(&q.bd);
    r.dmin = ld_rec<COH>(&q.dmin); r.dmax = ld_rec<COH>(&q.dmax);
  }
  return r;
}

template <typename E, bool COH>
__device__ __forceinline__ void wave_pick(const Params& P, int b, const Draw& w, const FinPart& r,
                                          int lane) {
  const int nF = P.nF;
  const FinPart* fp = P.fpart + size_t(b) * nF;
  double* xmass = P.fmass + size_t(b) * nF;          // exact item masses of the slow path
  const E* trow = final_row<E>(P, b, w.j, false);
  const E* drow = w.residual ? final_row<E>(P, b, w.j, true) : trow;
  const bool one = nF <= 64;
  // the record of item f (f = lane + 64 k, this lane's)
  auto rec = [&](int f) {
    if (one) return r;
    FinPart x = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, INFINITY, -INFINITY};
    if (f < nF) {
      const FinPart& q = fp[f];
      x.st = ld_rec<COH>(&q.st); x.sd = ld_rec<COH>(&q.sd);
      x.at = ld_rec<COH>(&q.at); x.ad = ld_rec<COH>(&q.ad);
      x.bt = ld_rec<COH>(&q.bt); x.bd = ld_rec<COH>(&q.bd);
      x.dmin = ld_rec<COH>(&q.dmin); x.dmax = ld_rec<COH>(&q.dmax);
    }
    return x;
  };

  double st = 0.0, sd = 0.0;
  int multi = 0;
  for (int base = 0; base < nF; base += 64) {
    const FinPart x = rec(base + lane);
    st += x.st;
    sd += x.sd;
    if (x.dmin < x.dmax) multi = 1;
  }
  st = wave_total(st);
  sd = wave_total(sd);
  const double it = 1.0 / st, id = 1.0 / sd;
  // did the band hold the exact ratio (with room for the rounding of its bounds), and is every
  // item's in-band set one ratio class?
  const bool slow = w.residual &&
                    (__any(multi) || !(fabsf(ln_hw(float(st / sd)) - float(w.lnrho)) < 0.5f * float(kBand)));
  if (slow) {
    for (int f = 0; f < nF; ++f) {
      const double m = item_exact_mass<E>(P, trow, drow, w, f, false, it, id, lane);
      if (lane == 0) st_dev(xmass + f, m);
    }
    wait_stores();
  }
  bool target_only = !w.residual;
  // mass of item f: normalised residual, or unnormalised p (bonus draw, zero-mass fallback)
  auto mass = [&](int f) {
    if (f >= nF) return 0.0;
    if (slow && !target_only) return ld_dev(xmass + f);
    const FinPart x = rec(f);
    if (target_only) return x.st;
    double m = x.at * it - x.ad * id;
    if (x.dmin <= x.dmax) m += fmax(0.0, x.bt * it - x.bd * id);   // one in-band ratio class
    return fmax(0.0, m);
  };

  // Z, then the first item whose inclusive prefix exceeds t = u Z (else the last item with
  // positive mass), 64 items at a time (up to 64 items: one scan gives both)
  double Z = 0.0, t = 0.0;
  int fstar = -1, flast = -1;
  double run = 0.0;
  if (one) {
    double m = mass(lane);
    double inc = dpp_scan_add(m);
    Z = readlane(inc, 63);
    if (!(Z > 0.0) && !target_only) {
      target_only = true;              // residual of zero mass (rounding only): draw from p_j
      m = mass(lane);
      inc = dpp_scan_add(m);
      Z = readlane(inc, 63);
    }
    t = w.u * Z;
    const unsigned long long over = __ballot(lane < nF && inc > t);
    const unsigned long long pos = __ballot(lane < nF && m > 0.0);
    if (pos) flast = 63 - __builtin_clzll(pos);
    if (over) {
      fstar = __builtin_ctzll(over);
      run = readlane(inc - m, fstar);
    }
  } else {
    for (int base = 0; base < nF; base += 64) Z += wave_total(mass(base + lane));
    if (!(Z > 0.0) && !target_only) {
      target_only = true;
      Z = 0.0;
      for (int base = 0; base < nF; base += 64) Z += wave_total(mass(base + lane));
    }
    t = w.u * Z;
    double total = 0.0;
    for (int base = 0; base < nF && fstar < 0; base += 64) {
      const int f = base + lane;
      const double m = mass(f);
      const double inc = dpp_scan_add(m) + total;
      const unsigned long long over = __ballot(f < nF && inc > t);
      const unsigned long long pos = __ballot(f < nF && m > 0.0);
      if (pos) flast = base + 63 - __builtin_clzll(pos);
      if (over) {
        const int l = __builtin_ctzll(over);
        fstar = base + l;
        run = readlane(inc - m, l);
      }
      total = readlane(inc, 63);
    }
  }
  const bool past_end = fstar < 0;
  int32_t* out = P.out_tokens + size_t(b) * (P.D + 1) + w.j;
  if (past_end) {
    fstar = flast;
    if (fstar < 0) {                   // no positive weight at all
      if (lane == 0) *out = -1;
      return;
    }
  }

  // The chosen item's elements. Its block masses come from the item record when they can (no
  // in-band element, and the draw's weights are the ones the blocks summed); then only the block
  // holding t is rescanned, else every block in order.
  const int a0 = fstar * kItemElems<E>;
  ItemRuns<E> tr, dr;
  load_item<E>(tr, dr, trow, drow, !target_only, a0, P.V, lane);
  constexpr int KB = kItemBlocks<E>;
  const FinPart* rf = fp + fstar;
  const bool bonus = !w.residual;
  const bool blockwise = !past_end && !slow && (bonus || (!target_only &&
                         !(ld_rec<COH>(&rf->dmin) <= ld_rec<COH>(&rf->dmax))));
  int kfirst = 0, klast = KB - 1;
  if (blockwise) {
    double bm = 0.0;                   // lane k: mass of block k
    if (lane < KB) {
      const double ka = ld_rec<COH>(&rf->kat[lane]);
      bm = bonus ? ka : fmax(0.0, ka * it - ld_rec<COH>(&rf->kad[lane]) * id);
    }
    const double inc = dpp_scan_add(bm) + run;
    const unsigned long long over = __ballot(lane < KB && inc > t);
    if (over) {                        // else rounding: rescan every block
      kfirst = klast = __builtin_ctzll(over);
      run = readlane(inc - bm, kfirst);
    }
  }
  int found = -1, last_pos = -1;
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    if (found < 0 && k >= kfirst && k <= klast) {     // wave-uniform
      const int a = a0 + kFinBlock * k + kFinPer * lane;
      const int n = max(0, min(kFinPer, P.V - a));
      double ls = 0.0, wts[kFinPer];
      if (n == kFinPer) {              // full run: no per-element branches, eight independent chains
#pragma unroll
        for (int e = 0; e < kFinPer; ++e)
          wts[e] = exact_weight<E>(tr.r[k], dr.r[k], e, w, target_only, it, id);
      } else {
#pragma unroll
        for (int e = 0; e < kFinPer; ++e)
          wts[e] = e < n ? exact_weight<E>(tr.r[k], dr.r[k], e, w, target_only, it, id) : 0.0;
      }
#pragma unroll
      for (int e = 0; e < kFinPer; ++e) {
        ls += wts[e];
        if (wts[e] > 0.0) last_pos = a + e;
      }
      const double inc = dpp_scan_add(ls) + run;
      // lane l owns [prefix before l, prefix through l): consecutive stored values, one owner
      const double mylo = lane_before(inc, run);
      const bool owner = !past_end && ls > 0.0 && mylo <= t && t < inc;
      const unsigned long long own = __ballot(owner);
      if (own) {
        const int ol = __builtin_ctzll(own);
        int k2 = -1;
        if (lane == ol) {
          double acc = mylo;
          int my_last = -1;
#pragma unroll
          for (int e = 0; e < kFinPer; ++e) {
            if (e < n && k2 < 0) {
              acc += wts[e];
              if (wts[e] > 0.0) my_last = a + e;
              if (acc > t) k2 = a + e;
            }
          }
          if (k2 < 0) k2 = my_last;    // rounding: the lane's last element of positive weight
        }
        found = __builtin_amdgcn_readlane(k2, ol);
      }
      run = readlane(inc, 63);
    }
  }
  if (found < 0) {                     // rounding put u * Z past the end: the last element
    for (int off = 32; off > 0; off >>= 1)   // with positive weight
      last_pos = max(last_pos, __shfl_xor(last_pos, off));
  }
  if (lane == 0) *out = (found >= 0) ? found : last_pos;
}

// Main sweep of an item: per block, the sum of e_t (bonus draws) or the sums of e_t and e_d
// over the elements above the band (residual draws, which also sum e_t and e_d over all
// elements); returns whether any of the lane's elements lies inside the band.
// FULL: every element of the item exists (all items but a row's last).
template <typename E, bool FULL, bool RES>
__device__ __forceinline__ bool item_sweep(const Params& P, int a0, const Draw& w,
                                           const ItemRuns<E>& tr, const ItemRuns<E>& dr,
                                           int lane, double& st, double& sd, double* kat,
                                           double* kad) {
  int band = 0;
#pragma unroll
  for (int k = 0; k < kItemBlocks<E>; ++k) {
    const int n = FULL ? kFinPer : max(0, min(kFinPer, P.V - (a0 + kFinBlock * k + kFinPer * lane)));
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) {
      if (FULL || e < n) {
        const double xt = tr.r[k].at(e);
        const double et = w.t(float(xt));
        if (RES) {
          st += et;
          const double xd = dr.r[k].at(e);
          const double ed = w.d(float(xd));
          sd += ed;
          // x_t - x_d against the band: above it the element is certainly in the positive part
          const double dx = xt - xd;
          const bool le = dx <= w.dhi;
          const double above = le ? 0.0 : 1.0;
          kat[k] = fma(above, et, kat[k]);
          kad[k] = fma(above, ed, kad[k]);
          band |= int(le) & int(dx >= w.dlo);               // no branch per element
        } else {
          kat[k] += et;
        }
      }
    }
    // blocks in order: block k + 1's data is not touched before block k is summed, so the
    // wavefront starts on a block as soon as its loads have landed
    __builtin_amdgcn_sched_barrier(0);
  }
  return band != 0;
}

// fp64 partial sums of item f of sequence b (the lane loads its runs), stored to the item's
// record. The rare elements inside the band are summed by a second sweep, taken only by
// wavefronts that have some.
template <typename E>
__device__ __forceinline__ void item_sums(const Params& P, int b, int f, const Draw& w,
                                          int lane) {
  constexpr int KB = kItemBlocks<E>;
  const int a0 = f * kItemElems<E>;
  const E* trow = final_row<E>(P, b, w.j, false);
  const E* drow = final_row<E>(P, b, w.j, true);
  // Items of full length whose rows are 16-byte aligned load with straight-line vector loads,
  // block by block, so that the sweep of a block waits only for that block's data.
  const uintptr_t bases = reinterpret_cast<uintptr_t>(trow) |
                          (w.residual ? reinterpret_cast<uintptr_t>(drow) : uintptr_t(0));
  const bool fast = a0 + kItemElems<E> <= P.V && (bases & 15) == 0;
  double st = 0, sd = 0, bt = 0, bd = 0, dmin = INFINITY, dmax = -INFINITY;
  double kat[KB], kad[KB];
#pragma unroll
  for (int k = 0; k < KB; ++k) kat[k] = kad[k] = 0.0;
  bool band;
  ItemRuns<E> tr, dr;
  if (w.residual) {
    if (fast) {
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int a = a0 + kFinBlock * k + kFinPer * lane;
        tr.r[k].load_vec(trow + a);
        dr.r[k].load_vec(drow + a);
      }
      __builtin_amdgcn_sched_barrier(0);          // every load issued before the sweep
      band = item_sweep<E, true, true>(P, a0, w, tr, dr, lane, st, sd, kat, kad);
    } else {
      load_item<E>(tr, dr, trow, drow, true, a0, P.V, lane);
      band = item_sweep<E, false, true>(P, a0, w, tr, dr, lane, st, sd, kat, kad);
    }
  } else {
    if (fast) {
#pragma unroll
      for (int k = 0; k < KB; ++k) tr.r[k].load_vec(trow + a0 + kFinBlock * k + kFinPer * lane);
      __builtin_amdgcn_sched_barrier(0);
      band = item_sweep<E, true, false>(P, a0, w, tr, dr, lane, st, sd, kat, kad);
    } else {
      load_item<E>(tr, dr, trow, drow, false, a0, P.V, lane);
      band = item_sweep<E, false, false>(P, a0, w, tr, dr, lane, st, sd, kat, kad);
    }
  }
  const bool any_band = __any(band);
  if (any_band) {                      // rare: reload the item and sum its in-band elements
    for (int k = 0; k < KB; ++k) {
      const int a = a0 + kFinBlock * k + kFinPer * lane;
      const int n = max(0, min(kFinPer, P.V - a));
      for (int e = 0; e < n; ++e) {
        const double xt = Elem<E>::get(trow, size_t(a + e));
        const double xd = Elem<E>::get(drow, size_t(a + e));
        const double dx = xt - xd;
        if (dx <= w.dhi && dx >= w.dlo) {
          bt += w.t(float(xt));
          bd += w.d(float(xd));
          dmin = fmin(dmin, dx);
          dmax = fmax(dmax, dx);
        }
      }
    }
  }
  const auto mn = [](double u, double v) { return fmin(u, v); };
  const auto mx = [](double u, double v) { return fmax(u, v); };
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    kat[k] = dpp_scan_add(kat[k]);
    if (w.residual) kad[k] = dpp_scan_add(kad[k]);
  }
  if (w.residual) {
    st = dpp_scan_add(st);
    sd = dpp_scan_add(sd);
    if (any_band) {                    // else every lane holds the identities already
      bt = dpp_scan_add(bt);
      bd = dpp_scan_add(bd);
      dmin = dpp_scan(dmin, INFINITY, mn);
      dmax = dpp_scan(dmax, -INFINITY, mx);
    }
  }
  if (lane == 63) {
    double at = 0.0, ad = 0.0, et = 0.0;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      at += kat[k];
      ad += kad[k];
    }
    if (!w.residual) et = at;          // bonus draw: the block sums are sums of e_t
    FinPart* q = P.fpart + size_t(b) * P.nF + f;
    FinPart x;
    x.st = w.residual ? st : et; x.sd = sd; x.at = at; x.ad = ad;
    x.bt = bt; x.bd = bd; x.dmin = dmin; x.dmax = dmax;
#pragma unroll
    for (int k = 0; k < kMaxItemBlocks; ++k) {
      x.kat[k] = k < KB ? kat[k] : 0.0;
      x.kad[k] = k < KB ? kad[k] : 0.0;
    }
    if (P.merged) {                    // a pick in this kernel reads it
      const double* src = reinterpret_cast<const double*>(&x);
      double* dst = reinterpret_cast<double*>(q);
#pragma unroll
      for (int i = 0; i < int(sizeof(FinPart) / sizeof(double)); ++i) st_dev(dst + i, src[i]);
    } else {
      *q = x;
    }
  }
}

__device__ inline unsigned long long uniform64(unsigned long long v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane(unsigned(v));
  const unsigned hi = __builtin_amdgcn_readfirstlane(unsigned(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// Does a sequence's outcome pair (a, c) call for a final draw?
__device__ inline bool draw_ready(unsigned long long a, unsigned long long c) {
  return unsigned(a & 3u) >= kResidual && ((c >> 32) & 1u);
}

// ------------------------------------------------------------------------------------------
// workgroups

// Grid (nchunk, 2 nb, D+1), dispatched x fastest: position-major; within a position the target
// rows of every sequence, then the draft rows (measured faster than alternating target and
// draft rows per sequence); chunks of a row consecutive.
template <typename E>
__device__ __forceinline__ void row_workgroup(const Params& P, Shared& sm, int tid) {
  const int c = int(blockIdx.x);
  const int which = int(blockIdx.y) >= P.nb ? 1 : 0;  // 0 target row p, 1 draft row p
  const int b = P.b0 + int(blockIdx.y) - which * P.nb;
  const int p = P.p_lo + int(blockIdx.z);
  const int D = P.D;
  if (P.merged && p == 0 && which == 0 && c == 0 && tid == 0)
    P.done[b] = 0u;                                   // the item kernel counts from zero
  const int L = P.lens ? P.lens[b] : D;
  const float T = P.temperature[b];
  if (!seq_valid(L, D, T)) return;    // invalid length or temperature: nothing is read
  if (P.dead && unsigned(p) > P.dead[b]) return;   // past a known rejection: not needed
  const bool greedy = (T == 0.f);
  if (which == 0 ? (p <= L) : (!greedy && !P.thresh && p < L))   // rows the method needs
    row_chunk<E>(P, sm, b, p, which, c, L, T, greedy, tid);
}

// Final-draw item wavefront: item f of sequence b (wave-uniform), after the row kernel, given
// the sequence's outcome.
template <typename E>
__device__ __forceinline__ void item_wavefront(const Params& P, const double* e2, int b, int f,
                                               const Outcome& o, int lane) {
  if (o.mode != kResidual && o.mode != kBonus) return;   // no draw (greedy or invalid)
  item_sums<E>(P, b, f, make_draw(P, b, o, e2), lane);
}

// Pick wavefront of sequence b < B, after every item is stored, with its first item records r
// and outcome words (a, c) loaded.
template <typename E>
__device__ __forceinline__ void pick_wavefront(const Params& P, const double* e2, int b,
                                               const FinPart& r, unsigned long long a,
                                               unsigned long long c, int lane) {
  if (!draw_ready(a, c)) return;
  const Outcome o = {unsigned(a & 3u), int((a >> 2) & 31u), __uint_as_float(unsigned(a >> 32)),
                     __uint_as_float(unsigned(c)), __uint_as_float(unsigned(c >> 32)),
                     P.uniforms[size_t(b) * (P.D + 1) + P.D]};
  wave_pick<E, false>(P, b, make_draw(P, b, o, e2), r, lane);
}

// ------------------------------------------------------------------------------------------
// the kernels

// Row kernel: one workgroup per row chunk.
template <typename E>
__global__ __launch_bounds__(kThreads) void row_kernel(Params P) {
  __shared__ Shared sm;
  row_workgroup<E>(P, sm, threadIdx.x);
}

// Final-draw kernels, after the row kernel: outcome and partial sums (one wavefront per item),
// then the pick (one wavefront per sequence).
// Item kernel: the kWaves wavefronts of a workgroup take consecutive items of one sequence
// (items per sequence rounded up to a multiple of kWaves; the extra ones do nothing).
// Wavefront 0 derives the sequence's outcome (and, for the sequence's first workgroup, writes
// it) while the others fill the e2 table; the outcome reaches them through LDS.
template <typename E>
__global__ __launch_bounds__(kThreads) void item_kernel(Params P) {
  __shared__ double e2[256];
  __shared__ Outcome so;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int per_seq = int(gridDim.x);                     // workgroups per sequence
  const int b = P.b0 + int(blockIdx.y);
  const int f = int(blockIdx.x) * kWaves + wave;
  if (wave == 0) {
    if (P.pre) {                       // stored by the outcome kernel
      const unsigned long long a = uniform64(P.pub[b].a);
      const unsigned long long c = uniform64(P.pub[b].c);
      if (lane == 0)
        so = Outcome{unsigned(a & 3u), int((a >> 2) & 31u), __uint_as_float(unsigned(a >> 32)),
                     __uint_as_float(unsigned(c)), __uint_as_float(unsigned(c >> 32)),
                     P.uniforms[size_t(b) * (P.D + 1) + P.D]};
    } else {
      const OutcomeIn in = load_outcome(P, b, lane);
      const Outcome o = seq_outcome<E>(P, b, in, lane, f == 0);
      if (lane == 0) so = o;
    }
  }
  fill_e2(e2, tid);
  __syncthreads();
  Outcome o;                           // wave-uniform copies of the shared words
  o.mode = unsigned(uniform(int(so.mode)));
  o.j = uniform(so.j);
  o.mt = __int_as_float(uniform(__float_as_int(so.mt)));
  o.md = __int_as_float(uniform(__float_as_int(so.md)));
  o.lnrho = __int_as_float(uniform(__float_as_int(so.lnrho)));
  o.u = __int_as_float(uniform(__float_as_int(so.u)));
  if (f < P.nF) item_wavefront<E>(P, e2, b, f, o, lane);
  if (!P.merged || (o.mode != kResidual && o.mode != kBonus)) return;
  // The workgroup that completes the sequence's last items picks its token: each wavefront's
  // record stores complete, then one count per workgroup.
  __shared__ unsigned last;
  wait_stores();
  __syncthreads();
  if (tid == 0) last = add_dev(P.done + b, 1u) == unsigned(per_seq - 1) ? 1u : 0u;
  __syncthreads();
  if (wave != 0 || last == 0u) return;
  wave_pick<E, true>(P, b, make_draw(P, b, o, e2), first_records<true>(P, b, lane), lane);
}

// Outcome kernel (item grids of more than one round only): one wavefront per sequence derives
// the outcome once and stores AL, the tokens other than the final draw's and the outcome words,
// so that each of the sequence's item workgroups starts from one load rather than from the row
// partials.
template <typename E>
__global__ __launch_bounds__(kThreads) void outcome_kernel(Params P) {
  const int lane = threadIdx.x & 63;
  const int b = int(blockIdx.x) * kWaves + uniform(int(threadIdx.x >> 6));
  if (b >= P.B) return;
  const OutcomeIn in = load_outcome(P, b, lane);
  (void)seq_outcome<E>(P, b, in, lane, true);
}

// Decision kernel between staged row launches: one wavefront per sequence evaluates the
// positions below `limit` (their rows are all read) exactly as the outcome does, and stores the
// first of them that rejects (0xffffffff if none does; 0 for a row already marked invalid), so
// that the next launches do not read the rows past it.
template <typename E>
__global__ __launch_bounds__(kThreads) void decide_kernel(Params P, int limit, unsigned* dead) {
  const int lane = threadIdx.x & 63;
  const int b = int(blockIdx.x) * kWaves + uniform(int(threadIdx.x >> 6));
  if (b >= P.B) return;
  const int L = P.lens ? P.lens[b] : P.D;
  const float T = P.temperature[b];
  unsigned d = 0u;
  if (seq_valid(L, P.D, T)) {
    const OutcomeIn in = load_outcome(P, b, lane);
    const Outcome o = seq_outcome<E>(P, b, in, lane, false, limit);
    d = (o.j < min(L, limit)) ? unsigned(o.j) : 0xffffffffu;
  }
  if (lane == 0) dead[b] = d;
}

template <typename E>
__global__ __launch_bounds__(kThreads) void pick_kernel(Params P) {
  __shared__ double e2[256];
  const int tid = threadIdx.x, lane = tid & 63;
  fill_e2(e2, tid);
  __syncthreads();
  const int b = int(blockIdx.x) * kWaves + uniform(tid >> 6);
  if (b >= P.B) return;
  const FinPart r = first_records<false>(P, b, lane);
  const unsigned long long a = uniform64(P.pub[b].a);
  const unsigned long long c = uniform64(P.pub[b].c);
  pick_wavefront<E>(P, e2, b, r, a, c, lane);
}

// ------------------------------------------------------------------------------------------
// host side

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Final-draw item length for a dtype: kItemsPerChunk items per row chunk, 4 KB of each final
// row (2048 bf16 or 1024 fp32 logits, four blocks of 512): one wavefront's item. Half as long
// measured slower (twice the items for every pick), twice as long needs more registers.
inline int item_elems(int elem_bytes) { return kRowChunkBytes / elem_bytes / kItemsPerChunk; }

// Workspace: [outcome words B][row partials][final-draw partials][pick scratch][item counters B].
// Every part is written before it is read within one call (the row kernel zeroes the counters),
// so a workspace needs no initialisation. One
// layout serves both dtypes (nF and nchunk are those of the dtype with more).
struct Layout {
  int nchunk, nF;
  size_t off_pub, off_rpart, off_fpart, off_fmass, off_done, off_dead, total;
};

inline bool make_layout(int B, int D, int V, Layout& L) {
  if (B <= 0 || D < 0 || V <= 0 || D > SV_MAX_D) return false;
  const int rch = kRowChunkBytes / 4, fch = item_elems(4);      // fp32: the most chunks/items
  L.nchunk = int((size_t(V) + rch - 1) / rch);
  L.nF = int((size_t(V) + fch - 1) / fch);
  const size_t R = size_t(2) * D + 1;
  size_t o = 0;
  L.off_pub = o;   o += align256(size_t(B) * sizeof(SeqPub));
  L.off_rpart = o; o += align256(size_t(B) * R * L.nchunk * sizeof(RowPart));
  L.off_fpart = o; o += align256(size_t(B) * L.nF * sizeof(FinPart));
  L.off_fmass = o; o += align256(size_t(B) * L.nF * sizeof(double));
  L.off_done = o;  o += align256(size_t(B) * sizeof(unsigned));
  L.off_dead = o;  o += align256(size_t(B) * sizeof(unsigned));
  L.total = o;
  return true;
}

inline size_t workspace_bytes(int B, int D, int V) {
  Layout a;
  return make_layout(B, D, V, a) ? a.total : 0;
}

struct DeviceWorkspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};

// Library-owned workspaces of the plain entry points: one per (device, stream) that has called
// them, grown in stream order (hipMallocAsync / hipFreeAsync: the host never waits) and held
// until spec_verify_release(stream) or the end of the process.
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, DeviceWorkspace> g_ws;

struct Profile {        // optional timing of the row kernel: one event pair per row launch
  std::vector<hipEvent_t> begin, end;
  int used = 0;
  bool armed = false;
};
std::mutex g_prof_mutex;
Profile g_prof;

// Scratch of the entry point that allocates nothing (spec_verify_noalloc): file-scope device
// memory of a fixed size, one copy on every GPU the library runs on, held until the process
// ends. In host code `scratch` only names the symbol; its device address on the current device
// comes from hipGetSymbolAddress, taken once per device and kept here. Every call on a device
// shares that device's copy, so calls that overlap on one GPU race (each call writes every part
// of it that it reads, so nothing needs clearing between calls).
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
std::map<int, void*> g_scratch;      // device -> device address of that device's scratch

int scratch_address(void** out) {
  int dev = 0, count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return SV_ENODEV;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ENODEV;
  std::lock_guard<std::mutex> g(g_scratch_mutex);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return SV_EHIP;
    it = g_scratch.emplace(dev, p).first;
  }
  *out = it->second;
  return SV_OK;
}

int check_args(const void* t, const void* d, const int32_t* tok, const float* u, const float* temp,
               int32_t* ol, int32_t* ot, int B, int D, int V, bool need_draft = true) {
  if (B <= 0 || D < 0 || V <= 0 || D > SV_MAX_D) return SV_EINVAL;
  if (!t || !u || !temp || !ol || !ot) return SV_EINVAL;
  if (D > 0 && ((need_draft && !d) || !tok)) return SV_EINVAL;
  const unsigned __int128 n = (unsigned __int128)B * (unsigned __int128)(D + 1) * (unsigned __int128)V;
  if (n > ((unsigned __int128)1 << 60)) return SV_EINVAL;
  return SV_OK;
}

// Row launches of a call: stage s reads positions [cuts[s], cuts[s + 1]). One stage when staging
// is off (debug exports, which report every row), for D = 0, or when the rows are too few for a
// stage boundary (a decision kernel and a second row launch, about 7 us) to pay; else a cut at
// position 1 for D = 1, at 2 for D <= 3 or up to 512 MB of rows, at 1 and 3 beyond. Returns the
// number of stages.
constexpr int kMaxStages = 3;
constexpr size_t kStageMinBytes = size_t(64) << 20, kStageTwoCutBytes = size_t(512) << 20;
inline int stage_plan(bool stage, int B, int D, int V, int elem_bytes, int* cuts) {
  const int npos = D + 1;
  const size_t bytes = size_t(B) * size_t(2 * D + 1) * size_t(V) * size_t(elem_bytes);
  int n = 0;
  cuts[n++] = 0;
  if (stage && npos >= 2 && bytes >= kStageMinBytes) {
    if (npos == 2) {
      cuts[n++] = 1;
    } else if (npos <= 4 || bytes <= kStageTwoCutBytes) {
      cuts[n++] = 2;
    } else {
      cuts[n++] = 1;
      cuts[n++] = 3;
    }
  }
  cuts[n] = npos;
  return n;
}

// Item workgroups resident at once on the current device (0 if unknown).
template <typename E>
long long item_capacity() {
  static std::mutex m;
  static std::map<int, long long> cap;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> g(m);
  auto it = cap.find(dev);
  if (it != cap.end()) return it->second;
  int per_cu = 0, cus = 0;
  long long c = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, item_kernel<E>, kThreads, 0) ==
          hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    c = (long long)per_cu * cus;
  cap[dev] = c;
  return c;
}

template <typename E>
int launch(Params& P, hipStream_t stream) {
  const long long rows = (long long)(P.D + 1) * P.B * 2 * P.nchunk;
  const long long items = (long long)P.B * ((P.nF + kWaves - 1) / kWaves);
  const long long picks = ((long long)P.B + kWaves - 1) / kWaves;
  if (rows > 0x7fffffffll || items > 0x7fffffffll) return SV_EINVAL;
  // When every item workgroup is resident at once, the last one of each sequence picks its
  // token (no pick kernel); otherwise a count would hold slots that later items need.
  P.merged = items <= item_capacity<E>() ? 1 : 0;
  // More than one round of item workgroups: derive each outcome once, in its own kernel (one
  // round, one wavefront per sequence), rather than once per item workgroup.
  P.pre = P.merged ? 0 : 1;

  // A grid's y dimension holds at most 65535 workgroups: larger batches launch in slices of
  // sequences (stream-ordered, so each kernel still sees every earlier kernel's results).
  constexpr int kRowSlice = 32767, kItemSlice = 65535;
  // Timing (profile hook armed): each row launch takes an event pair as its own start and end
  // stamps.
  // Staged row launches (stage_plan), each after the first preceded by the decision kernel
  // for the positions read so far, so that the rows past a known rejection are not read.
  int cuts[kMaxStages + 1];
  const int ncut = stage_plan(P.stage != 0, P.B, P.D, P.V, int(sizeof(E)), cuts);
  for (int st = 0; st < ncut; ++st) {
    if (st > 0) {
      Params Q = P;
      Q.b0 = 0;
      Q.nb = P.B;
      hipLaunchKernelGGL(decide_kernel<E>, dim3(unsigned(picks)), dim3(kThreads), 0, stream, Q,
                         cuts[st], P.dead_buf);
      if (hipGetLastError() != hipSuccess) return SV_EHIP;
    }
    for (int b0 = 0; b0 < P.B; b0 += kRowSlice) {
      Params Q = P;
      Q.b0 = b0;
      Q.nb = std::min(kRowSlice, P.B - b0);
      Q.p_lo = cuts[st];
      Q.dead = st > 0 ? P.dead_buf : nullptr;
      // threshold acceptance reads no draft row: the grid holds the target rows only
      const dim3 grid(unsigned(Q.nchunk), unsigned((Q.thresh ? 1 : 2) * Q.nb),
                      unsigned(cuts[st + 1] - cuts[st]));
      hipEvent_t ev0 = nullptr, ev1 = nullptr;
      {
        std::lock_guard<std::mutex> g(g_prof_mutex);
        if (g_prof.armed && g_prof.used < int(g_prof.begin.size())) {
          ev0 = g_prof.begin[size_t(g_prof.used)];
          ev1 = g_prof.end[size_t(g_prof.used)];
          ++g_prof.used;
        }
      }
      if (ev0) {
        void* args[] = {&Q};
        if (hipExtLaunchKernel(reinterpret_cast<const void*>(&row_kernel<E>), grid,
                               dim3(kThreads), args, 0, stream, ev0, ev1, 0) != hipSuccess)
          return SV_EHIP;
      } else {
        hipLaunchKernelGGL(row_kernel<E>, grid, dim3(kThreads), 0, stream, Q);
        if (hipGetLastError() != hipSuccess) return SV_EHIP;
      }
    }
  }
  if (P.pre) {
    hipLaunchKernelGGL(outcome_kernel<E>, dim3(unsigned(picks)), dim3(kThreads), 0, stream, P);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
  }
  for (int b0 = 0; b0 < P.B; b0 += kItemSlice) {
    Params Q = P;
    Q.b0 = b0;
    Q.nb = std::min(kItemSlice, P.B - b0);
    hipLaunchKernelGGL(item_kernel<E>, dim3(unsigned((Q.nF + kWaves - 1) / kWaves), unsigned(Q.nb)),
                       dim3(kThreads), 0, stream, Q);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
  }
  if (!P.merged) {
    hipLaunchKernelGGL(pick_kernel<E>, dim3(unsigned(picks)), dim3(kThreads), 0, stream, P);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
  }
  return SV_OK;
}

int run(int dtype, const void* target, const void* draft, const int32_t* tokens,
        const int32_t* lens, const float* uniforms, int B, int D, int V, const float* temperature,
        int32_t* out_len, int32_t* out_tokens, void* ws, size_t ws_bytes, float* dbg_stats,
        int32_t* dbg_argmax, float* dbg_logpq, hipStream_t stream, bool thresh = false,
        double log_tau = 0.0) {
  if (dtype != 0 && dtype != 1) return SV_EDTYPE;
  int rc = check_args(target, draft, tokens, uniforms, temperature, out_len, out_tokens, B, D, V,
                      !thresh);
  if (rc != SV_OK) return rc;
  Layout lay;
  make_layout(B, D, V, lay);
  const int elem_bytes = dtype == 1 ? 2 : 4;
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
      // A stream under graph capture would record the allocation into the graph: growth is
      // refused there (a first call outside the capture, or spec_verify_ws, avoids it).
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return SV_EHIP;
      if (cap != hipStreamCaptureStatusNone) return SV_ENOMEM;
      // Stream-ordered: the old buffer is released after this stream's earlier calls have run,
      // the new one is ready for this call's kernels, and the host does not wait.
      if (w.ptr && hipFreeAsync(w.ptr, stream) != hipSuccess) return SV_EHIP;
      w.ptr = nullptr;
      w.bytes = 0;
      if (hipMallocAsync(&w.ptr, need, stream) != hipSuccess) { w.ptr = nullptr; return SV_ENOMEM; }
      w.bytes = need;
    }
    ws = w.ptr;
  }
  char* base = static_cast<char*>(ws);

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
  P.rch = kRowChunkBytes / elem_bytes;
  P.nchunk = int((size_t(V) + P.rch - 1) / P.rch);
  P.fch = item_elems(elem_bytes);
  P.nF = int((size_t(V) + P.fch - 1) / P.fch);
  P.pub = reinterpret_cast<SeqPub*>(base + lay.off_pub);
  P.rpart = reinterpret_cast<RowPart*>(base + lay.off_rpart);
  P.fpart = reinterpret_cast<FinPart*>(base + lay.off_fpart);
  P.fmass = reinterpret_cast<double*>(base + lay.off_fmass);
  P.done = reinterpret_cast<unsigned*>(base + lay.off_done);
  P.dead_buf = reinterpret_cast<unsigned*>(base + lay.off_dead);
  P.thresh = thresh ? 1 : 0;
  P.log_tau = log_tau;
  P.stage = (dbg_stats || dbg_argmax || dbg_logpq) ? 0 : 1;
  P.dbg_row_stats = dbg_stats;
  P.dbg_argmax = dbg_argmax;
  P.dbg_logpq = dbg_logpq;
  if (dbg_stats && hipMemsetAsync(dbg_stats, 0xff, size_t(B) * P.R * 2 * 4, stream) != hipSuccess)
    return SV_EHIP;                    // 0xffffffff: NaN for rows that are never evaluated
  if (dbg_argmax && hipMemsetAsync(dbg_argmax, 0xff, size_t(B) * (D + 1) * 4, stream) != hipSuccess)
    return SV_EHIP;                    // -1
  if (dbg_logpq && D > 0 && hipMemsetAsync(dbg_logpq, 0xff, size_t(B) * D * 2 * 4, stream) != hipSuccess)
    return SV_EHIP;
  return dtype == 1 ? launch<uint16_t>(P, stream) : launch<float>(P, stream);
}

// Epilogue after verification ("Accélérer Sonar par la Spéculation", section "Calendrier MTP
// pour un jeton unique": the input tokens are shifted and a kernel writes the new tokens into
// their slots, with no host synchronisation). One wavefront per sequence: its window of the W
// most recent tokens moves AL places and the AL emitted tokens fill the last slots; the length
// grows by AL. The window is updated in place, 64 slots per pass in ascending order: slot j
// takes slot j + AL (always a later slot) or an emitted token, and every lane's loads of a pass
// complete before that pass's stores (the stored values are the loaded ones), so no slot is
// overwritten before it has been read.
__global__ void __launch_bounds__(kThreads) advance_kernel(const int32_t* __restrict__ accept_len,
                                                           const int32_t* __restrict__ tokens,
                                                           int B, int D, int32_t* input_ids,
                                                           int W, int32_t* seq_len) {
  const int lane = int(threadIdx.x) & 63;
  const int b = int(blockIdx.x) * kWaves + int(threadIdx.x >> 6);
  if (b >= B) return;
  const int a = accept_len[b];
  const int n = seq_len ? seq_len[b] : 0;
  if (a < 1 || a > D + 1) return;
  if (seq_len && (n < 0 || n > 0x7fffffff - a)) return;
  int32_t* row = input_ids + size_t(b) * size_t(W);
  const int32_t* emitted = tokens + size_t(b) * size_t(D + 1);
  for (int j0 = 0; j0 < W; j0 += 64) {
    const int j = j0 + lane;
    if (j < W) {
      const int src = j + a;
      const int v = src < W ? row[src] : emitted[src - W];
      row[j] = v;
    }
  }
  if (seq_len && lane == 0) seq_len[b] = n + a;
}

// Saguaro draft reshaping ("Speculative Speculative Decoding - асинхронизируй это", saguaro
// sampling: the draft's most likely tokens get their probabilities lowered when the draft is
// generated). For each needed draft row (sampled sequence, position < L_b) the k largest logits
// (ties: lowest index) move by delta = T ln c, which multiplies their probabilities under q by c
// before renormalisation.
//
// Each needed row is read once, in units of 8 KB, one wavefront per unit (the four wavefronts of
// a workgroup never wait for each other): the unit's top k candidates go to the workspace. A
// second kernel then takes, with one wavefront per row, the row's top k from its units'
// candidates by k rounds of a wavefront argmax and writes the k new logits.
constexpr int kMaxTopK = 8;

__device__ inline bool tk_better(float a, int ia, float b, int ib) {
  return ib < 0 || a > b || (a == b && ia < ib);
}

// A sorted (best first) list of at most kMaxTopK (value, index) pairs; index -1 = empty.
struct TopList {
  float v[kMaxTopK];
  int i[kMaxTopK];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) { v[j] = -INFINITY; i[j] = -1; }
  }
  __device__ __forceinline__ void insert(float x, int ix) {
    if (ix < 0 || !tk_better(x, ix, v[kMaxTopK - 1], i[kMaxTopK - 1])) return;
    float cx = x;
    int ci = ix;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (tk_better(cx, ci, v[j], i[j])) {
        const float t = v[j]; v[j] = cx; cx = t;
        const int u = i[j]; i[j] = ci; ci = u;
      }
    }
  }
  // k rounds of a wavefront argmax over the lists' heads; round r's winner is returned in lane
  // r (value, index; index -1 when the lists ran out).
  __device__ __forceinline__ void wave_top(int k, int lane, float& rv, int& ri) {
    rv = -INFINITY;
    ri = -1;
    for (int r = 0; r < k; ++r) {
      float hv = v[0];
      int hi = i[0];
      wave_am(hv, hi);
      if (hi >= 0 && i[0] == hi) {          // the owner (unique index) drops its head
#pragma unroll
        for (int j = 0; j + 1 < kMaxTopK; ++j) { v[j] = v[j + 1]; i[j] = i[j + 1]; }
        v[kMaxTopK - 1] = -INFINITY;
        i[kMaxTopK - 1] = -1;
      }
      if (lane == r) { rv = hv; ri = hi; }
    }
  }
};

__device__ inline unsigned long long pack_cand(float v, int i) {
  return ((unsigned long long)uint32_t(i) << 32) | __float_as_uint(v);
}

// One wavefront per unit of kSagUnitBytes of a row (a quarter of a 32 KB row chunk); the four
// wavefronts of a workgroup take consecutive units and never wait for each other.
constexpr int kSagUnitBytes = kRowChunkBytes / kWaves;
constexpr int kSagVecs = kSagUnitBytes / 16 / 64;          // 16-byte vectors per lane (8)
constexpr int kSagCap = 128;                               // hits a wavefront keeps in LDS
constexpr int kSagSlots = 16;                              // candidate slots per unit

// The k-th largest (k <= 8) of the eight maxima of the wavefront's groups of eight lanes, given
// each lane's value m (every lane gets it). Each group maximum is some lane's value, so at least
// k lanes hold a value at or above the result.
__device__ __forceinline__ float group_kth(float m, int k) {
  float g = fmaxf(m, dpp_float<0x111, 0xf>(m, -INFINITY));    // row_shr:1
  g = fmaxf(g, dpp_float<0x112, 0xf>(g, -INFINITY));           // row_shr:2
  g = fmaxf(g, dpp_float<0x114, 0xf>(g, -INFINITY));           // row_shr:4: lane 8q + 7
  float t8[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    t8[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), 8 * q + 7));
#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {           // odd-even transposition sort, descending
#pragma unroll
    for (int q = pass & 1; q + 1 < 8; q += 2) {
      const float h = fmaxf(t8[q], t8[q + 1]), l = fminf(t8[q], t8[q + 1]);
      t8[q] = h;
      t8[q + 1] = l;
    }
  }
  float kth = t8[0];
#pragma unroll
  for (int q = 1; q < 8; ++q)
    if (q == k - 1) kth = t8[q];
  return kth;
}

// The hits of a 16-byte aligned unit of n elements (PARTIAL: n may be below a full unit),
// appended to the wavefront's part of shared memory (at most kSagCap kept; their number is
// returned). The unit is held in registers: vector j of lane l holds unit elements
// (l + 64 j) kV + e. All loads are issued before any is used: whole vectors with 16-byte loads
// (a partial unit loads its last, partial vector element by element, and holds -inf past n). Threshold: each group of eight lanes' maximum, and thr = the
// k-th largest of the eight group maxima (k <= 8); k groups hold an element at or above it, so
// thr is at most the unit's k-th largest logit and the unit's top k are among its elements
// >= thr, the hits (appended in any order: ties go by index).
template <typename E, bool PARTIAL>
__device__ __forceinline__ int unit_hits(const E* ptr, int n, int a0, int k, int lane, int* nhit,
                                         float* hv, int* hi) {
  constexpr int kV = Elem<E>::kVec;
  const uint4* vp = reinterpret_cast<const uint4*>(ptr);
  uint4 buf[kSagVecs];
  if constexpr (!PARTIAL) {
#pragma unroll
    for (int j = 0; j < kSagVecs; ++j) buf[j] = load_stream(vp + lane + j * 64);
  } else {
    const int nvec = n / kV;                       // whole vectors
    const uint4 ninf = make_uint4(Elem<E>::kNegInf, Elem<E>::kNegInf, Elem<E>::kNegInf,
                                  Elem<E>::kNegInf);
#pragma unroll
    for (int j = 0; j < kSagVecs; ++j)
      buf[j] = nvec > 0 ? load_stream(vp + min(lane + j * 64, nvec - 1)) : ninf;
    // vectors past the end hold -inf (a repeated element must not count twice below)
#pragma unroll
    for (int j = 0; j < kSagVecs; ++j)
      if (lane + j * 64 >= nvec) buf[j] = ninf;
    const int rem = n - nvec * kV;                 // elements of the partial vector
    const int jp = (nvec - lane) >> 6;             // the partial vector is lane's vector jp
    if (rem > 0 && ((nvec - lane) & 63) == 0) {
      uint32_t w[4] = {Elem<E>::kNegInf, Elem<E>::kNegInf, Elem<E>::kNegInf, Elem<E>::kNegInf};
#pragma unroll
      for (int e = 0; e < kV; ++e) {
        if (e < rem) {
          const uint32_t x = sizeof(E) == 2
              ? uint32_t(ld_global(reinterpret_cast<const uint16_t*>(ptr) + nvec * kV + e))
              : __float_as_uint(ld_global(reinterpret_cast<const float*>(ptr) + nvec * kV + e));
          if (sizeof(E) == 2) w[e >> 1] = (w[e >> 1] & (0xffffu << ((1 - (e & 1)) * 16))) | (x << ((e & 1) * 16));
          else w[e] = x;
        }
      }
#pragma unroll
      for (int j = 0; j < kSagVecs; ++j)
        if (j == jp) buf[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);               // every load issued before any use
  // the lane's maximum (a packed max for bf16, exact below 2^121 in magnitude). Where it may
  // not be the maximum it is replaced by -inf: any value at most the lane's largest element
  // keeps thr below at most the unit's k-th largest logit (a lower thr only makes more hits).
  typename Elem<E>::Acc acc = Elem<E>::acc_init();
#pragma unroll
  for (int j = 0; j < kSagVecs; ++j) acc = Elem<E>::acc_add(acc, buf[j]);
  float mx = Elem<E>::acc_value(acc);
  if (!(fabsf(mx) < 0x1p121f)) mx = -INFINITY;
  const float thr = group_kth(mx, k);
  if (lane == 0) *nhit = 0;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < kSagVecs; ++j) {
    const int e0 = (lane + j * 64) * kV;
#pragma unroll
    for (int e = 0; e < kV; ++e) {
      const float x = Elem<E>::lane(buf[j], e);
      if ((!PARTIAL || e0 + e < n) && x >= thr) {
        const int q = atomicAdd(nhit, 1);
        if (q < kSagCap) { hv[q] = x; hi[q] = a0 + e0 + e; }
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  return __builtin_amdgcn_readfirstlane(*nhit);
}

// Every element of a unit that is not 16-byte aligned (rows whose byte length is not a multiple
// of 16) through the lanes' sorted lists; a lane's kV elements of one vector are loaded together.
template <typename E>
__device__ __forceinline__ void unit_scan(const E* ptr, int n, int a0, int lane, TopList& tl) {
  constexpr int kV = Elem<E>::kVec;
  for (int j = 0; (j * 64) * kV < n; ++j) {
    const int e0 = (lane + j * 64) * kV;
    float x[kV];
#pragma unroll
    for (int e = 0; e < kV; ++e) x[e] = Elem<E>::get(ptr, size_t(min(e0 + e, n - 1)));
#pragma unroll
    for (int e = 0; e < kV; ++e)
      if (e0 + e < n) tl.insert(x[e], a0 + e0 + e);
  }
}

// Candidates: one wavefront per unit stores, in the unit's kSagSlots slots of the workspace, a
// set of candidates that holds the unit's top k: its hits when they fit, else its top k (taken
// from the hits, or from every element when the unit is a row's last or the row is not 16-byte
// aligned).
template <typename E>
__global__ __launch_bounds__(kThreads) void reshape_kernel(const E* draft, const int32_t* lens,
                                                           const float* temperature, int b0,
                                                           int D, int V, int nunit, int k,
                                                           unsigned long long* cand) {
  __shared__ int s_nhit[kWaves];
  __shared__ float s_hv[kWaves][kSagCap];
  __shared__ int s_hi[kWaves][kSagCap];
  const int tid = int(threadIdx.x), lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int u = int(blockIdx.x) * kWaves + wave;   // unit of the row
  const int i = int(blockIdx.y);
  const int b = b0 + int(blockIdx.z);
  const int L = lens ? lens[b] : D;
  const float T = temperature[b];
  if (!seq_valid(L, D, T) || !(T > 0.f) || i >= L || u >= nunit) return;
  const size_t rid = size_t(b) * D + i;
  const E* row = draft + rid * size_t(V);
  constexpr int ue = kSagUnitBytes / int(sizeof(E));
  const int a0 = u * ue;
  const int n = min(ue, V - a0);
  const E* ptr = row + a0;
  // The unit's slots: up to kSagSlots candidates (empty slots: index -1) that include its top k.
  unsigned long long* slot = cand + (rid * size_t(nunit) + u) * kSagSlots;
  int nh = kSagCap + 1;
  const bool aligned = (reinterpret_cast<uintptr_t>(ptr) & 15) == 0;
  if (aligned && n == ue)
    nh = unit_hits<E, false>(ptr, n, a0, k, lane, &s_nhit[wave], s_hv[wave], s_hi[wave]);
  else if (aligned)
    nh = unit_hits<E, true>(ptr, n, a0, k, lane, &s_nhit[wave], s_hv[wave], s_hi[wave]);
  if (nh <= kSagSlots) {                           // the usual case: the hits themselves
    if (lane < kSagSlots)
      slot[lane] = lane < nh ? pack_cand(s_hv[wave][lane], s_hi[wave][lane]) : pack_cand(0.f, -1);
    return;
  }
  // more hits than slots (many equal logits), or an unaligned unit: its top k
  TopList tl;
  tl.clear();
  if (nh <= kSagCap) {
    for (int q = lane; q < nh; q += 64) tl.insert(s_hv[wave][q], s_hi[wave][q]);
  } else {
    unit_scan<E>(ptr, n, a0, lane, tl);
  }
  float cv;
  int ci;
  tl.wave_top(k, lane, cv, ci);
  if (lane < kSagSlots) slot[lane] = lane < k ? pack_cand(cv, ci) : pack_cand(0.f, -1);
}

// Merge: one wavefront per row takes the row's top k from its units' candidates and writes the
// k new logits (fp32 sum without contraction, then bf16 round-to-nearest-even for bf16 rows).
// Each lane's best candidate gives a threshold (group_kth: at most the row's k-th largest
// candidate); the candidates at or above it go to shared memory, and each of them finds its rank
// by comparing itself with all of them (value, then the lower index first); ranks below k are
// the row's top k in order. Rows with more candidates than one pass of eight per lane, or more
// of them at the threshold than shared memory holds, go through the lanes' sorted lists.
constexpr int kSagMergeCap = 256;

template <typename E>
__global__ __launch_bounds__(kThreads) void reshape_merge_kernel(E* draft, const int32_t* lens,
                                                                 const float* temperature,
                                                                 int b0, int nb, int D, int V,
                                                                 int nunit, float lnf, int k,
                                                                 const unsigned long long* cand) {
  __shared__ int s_n[kWaves];
  __shared__ unsigned long long s_c[kWaves][kSagMergeCap];
  __shared__ unsigned long long s_top[kWaves][kMaxTopK];
  const int lane = int(threadIdx.x) & 63;
  const int wave = uniform(int(threadIdx.x) >> 6);
  const int r = int(blockIdx.x) * kWaves + wave;   // row of the slice
  if (r >= nb * D) return;
  const int b = b0 + r / D, i = r % D;
  const int L = lens ? lens[b] : D;
  const float T = temperature[b];
  if (!seq_valid(L, D, T) || !(T > 0.f) || i >= L) return;
  const size_t rid = size_t(b) * D + i;
  const unsigned long long* rc = cand + rid * size_t(nunit) * kSagSlots;
  const int ncand = nunit * kSagSlots;
  float myv = 0.f;
  int mine = -1;
  bool done = false;
  if (ncand <= 8 * 64) {
    // lane l takes slots s l .. s l + s - 1, s = ceil(ncand / 64): the slots spread over every
    // lane, so that each group of eight lanes holds candidates and the k-th largest group max
    // (below which no candidate can be in the top k, whatever the grouping) is a real bound
    const int sp = (ncand + 63) >> 6;
    unsigned long long w[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int q = lane * sp + t;
      w[t] = (t < sp && q < ncand) ? rc[q] : pack_cand(0.f, -1);
    }
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (int(uint32_t(w[t] >> 32)) >= 0) m = fmaxf(m, __uint_as_float(uint32_t(w[t])));
    const float thr = group_kth(m, k);
    if (lane == 0) s_n[wave] = 0;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (int(uint32_t(w[t] >> 32)) >= 0 && __uint_as_float(uint32_t(w[t])) >= thr) {
        const int q = atomicAdd(&s_n[wave], 1);
        if (q < kSagMergeCap) s_c[wave][q] = w[t];
      }
    }
    __builtin_amdgcn_wave_barrier();
    const int nh = __builtin_amdgcn_readfirstlane(s_n[wave]);
    if (nh <= kSagMergeCap) {
      for (int h = lane; h < nh; h += 64) {
        const unsigned long long c = s_c[wave][h];
        const float cv = __uint_as_float(uint32_t(c));
        const int ci = int(uint32_t(c >> 32));
        int rank = 0;
        for (int g = 0; g < nh; ++g) {
          const unsigned long long o = s_c[wave][g];
          rank += tk_better(__uint_as_float(uint32_t(o)), int(uint32_t(o >> 32)), cv, ci) &&
                  int(uint32_t(o >> 32)) != ci;
        }
        if (rank < k) s_top[wave][rank] = c;
      }
      __builtin_amdgcn_wave_barrier();
      if (lane < k && lane < nh) {
        const unsigned long long c = s_top[wave][lane];
        myv = __uint_as_float(uint32_t(c));
        mine = int(uint32_t(c >> 32));
      }
      done = true;
    }
  }
  if (!done) {
    TopList tl;
    tl.clear();
    for (int q0 = 0; q0 < ncand; q0 += 8 * 64) {   // eight loads in flight per lane
      unsigned long long w[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int q = q0 + t * 64 + lane;
        w[t] = q < ncand ? rc[q] : pack_cand(0.f, -1);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t)
        tl.insert(__uint_as_float(uint32_t(w[t])), int(uint32_t(w[t] >> 32)));
    }
    tl.wave_top(k, lane, myv, mine);
  }
  if (lane < k && mine >= 0) {
    E* row = draft + rid * size_t(V);
    const float sum = __fadd_rn(myv, __fmul_rn(T, lnf));
    if constexpr (sizeof(E) == 2) {
      const uint32_t w = __float_as_uint(sum);
      row[mine] = E((w + 0x7fffu + ((w >> 16) & 1u)) >> 16);
    } else {
      row[mine] = E(sum);
    }
  }
}

// Workspace of the reshaping: the candidates [B*D][nunit][kSagSlots]; every slot the merge reads
// is written by the same call first, so it needs no initialisation. One layout serves both
// dtypes (the unit count is fp32's, the larger).
struct SagLayout {
  int nunit;
  size_t total;
};

inline bool sag_layout(int B, int D, int V, SagLayout& L) {
  if (B <= 0 || D < 0 || V <= 0 || D > SV_MAX_D) return false;
  const int ue32 = kSagUnitBytes / 4;
  L.nunit = int((size_t(V) + ue32 - 1) / ue32);
  L.total = align256(size_t(B) * size_t(D) * size_t(L.nunit) * kSagSlots *
                     sizeof(unsigned long long));
  if (L.total == 0) L.total = 256;
  return true;
}

inline size_t sag_workspace_bytes(int B, int D, int V) {
  SagLayout l;
  return sag_layout(B, D, V, l) ? l.total : 0;
}

// Library-owned reshaping workspaces, one per (device, stream), grown in stream order like the
// verification workspaces and held until spec_verify_release(stream).
std::map<std::pair<int, hipStream_t>, DeviceWorkspace> g_sag;

// ws == nullptr: the library-owned workspace of (device, stream).
int saguaro_reshape(int dtype, void* draft, const int32_t* lens, const float* temperature, int B,
                    int D, int V, float factor, int k, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  if (dtype != 0 && dtype != 1) return SV_EDTYPE;
  if (B <= 0 || D < 0 || V <= 0 || D > SV_MAX_D || k < 1 || k > kMaxTopK) return SV_EINVAL;
  if (!(factor > 0.f) || !(factor <= 1.f)) return SV_EINVAL;
  if (!temperature || (D > 0 && !draft)) return SV_EINVAL;
  if ((unsigned __int128)B * (unsigned __int128)(D + 1) * (unsigned __int128)V >
      ((unsigned __int128)1 << 60))
    return SV_EINVAL;
  int dev = 0, count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return SV_ENODEV;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ENODEV;
  if (D == 0) return SV_OK;
  SagLayout lay;
  sag_layout(B, D, V, lay);
  if (ws != nullptr && (ws_bytes < lay.total || (reinterpret_cast<uintptr_t>(ws) & 255)))
    return SV_ENOMEM;
  const int ue = dtype == 1 ? kSagUnitBytes / 2 : kSagUnitBytes / 4;
  const int nunit = int((size_t(V) + ue - 1) / ue);
  if (nunit > 0x7fffffff / 64) return SV_EINVAL;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if (ws == nullptr) {
    DeviceWorkspace& w = g_sag[{dev, stream}];
    if (w.bytes < lay.total) {
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return SV_EHIP;
      if (cap != hipStreamCaptureStatusNone) return SV_ENOMEM;
      if (w.ptr && hipFreeAsync(w.ptr, stream) != hipSuccess) return SV_EHIP;
      w.ptr = nullptr;
      w.bytes = 0;
      if (hipMallocAsync(&w.ptr, lay.total, stream) != hipSuccess) { w.ptr = nullptr; return SV_ENOMEM; }
      w.bytes = lay.total;
    }
    ws = w.ptr;
  }
  unsigned long long* cand = static_cast<unsigned long long*>(ws);
  const float lnf = float(std::log(double(factor)));
  const int kk = std::min(k, V);
  constexpr int kSlice = 65535;
  for (int b0 = 0; b0 < B; b0 += kSlice) {
    const int nb = std::min(kSlice, B - b0);
    const dim3 grid(unsigned((nunit + kWaves - 1) / kWaves), unsigned(D), unsigned(nb));
    const unsigned mgrid = unsigned((size_t(nb) * D + kWaves - 1) / kWaves);
    if (dtype == 1) {
      hipLaunchKernelGGL(reshape_kernel<uint16_t>, grid, dim3(kThreads), 0, stream,
                         static_cast<const uint16_t*>(draft), lens, temperature, b0, D, V, nunit,
                         kk, cand);
      hipLaunchKernelGGL(reshape_merge_kernel<uint16_t>, dim3(mgrid), dim3(kThreads), 0, stream,
                         static_cast<uint16_t*>(draft), lens, temperature, b0, nb, D, V, nunit,
                         lnf, kk, cand);
    } else {
      hipLaunchKernelGGL(reshape_kernel<float>, grid, dim3(kThreads), 0, stream,
                         static_cast<const float*>(draft), lens, temperature, b0, D, V, nunit,
                         kk, cand);
      hipLaunchKernelGGL(reshape_merge_kernel<float>, dim3(mgrid), dim3(kThreads), 0, stream,
                         static_cast<float*>(draft), lens, temperature, b0, nb, D, V, nunit, lnf,
                         kk, cand);
    }
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
  }
  return SV_OK;
}

int advance(const int32_t* accept_len, const int32_t* tokens, int B, int D, int32_t* input_ids,
            int W, int32_t* seq_len, hipStream_t stream) {
  if (B <= 0 || D < 0 || D > SV_MAX_D || W <= 0) return SV_EINVAL;
  if (!accept_len || !tokens || !input_ids) return SV_EINVAL;
  if ((unsigned long long)B * (unsigned long long)W > (1ull << 60)) return SV_EINVAL;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return SV_ENODEV;
  const unsigned groups = unsigned((B + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(advance_kernel, dim3(groups), dim3(kThreads), 0, stream, accept_len, tokens,
                     B, D, input_ids, W, seq_len);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
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

int spec_verify_noalloc(int dtype, const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const int32_t* draft_lens,
                        const float* uniforms, int B, int D, int V, const float* temperature,
                        int32_t* out_accept_len, int32_t* out_tokens, hipStream_t stream) {
  if (dtype != 0 && dtype != 1) return SV_EDTYPE;
  const int rc = sv::check_args(target_logits, draft_logits, draft_tokens, uniforms, temperature,
                                out_accept_len, out_tokens, B, D, V);
  if (rc != SV_OK) return rc;
  const size_t need = sv::workspace_bytes(B, D, V);
  if (need == 0 || need > size_t(SV_NOALLOC_SCRATCH_BYTES)) return SV_ESCRATCH;
  void* ws = nullptr;
  const int rs = sv::scratch_address(&ws);
  if (rs != SV_OK) return rs;
  return sv::run(dtype, target_logits, draft_logits, draft_tokens, draft_lens, uniforms, B, D,
                 V, temperature, out_accept_len, out_tokens, ws, size_t(SV_NOALLOC_SCRATCH_BYTES),
                 nullptr, nullptr, nullptr, stream);
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

int spec_verify_threshold(int dtype, const void* target_logits, const int32_t* draft_tokens,
                          const int32_t* draft_lens, const float* uniforms, int B, int D, int V,
                          const float* temperature, float tau, int32_t* out_accept_len,
                          int32_t* out_tokens, hipStream_t stream) {
  if (!(tau >= 0.f) || std::isinf(tau)) return SV_EINVAL;
  const double log_tau = tau > 0.f ? std::log(double(tau)) : -INFINITY;
  return sv::run(dtype, target_logits, nullptr, draft_tokens, draft_lens, uniforms, B, D, V,
                 temperature, out_accept_len, out_tokens, nullptr, 0, nullptr, nullptr, nullptr,
                 stream, true, log_tau);
}

int spec_verify_saguaro_reshape(int dtype, void* draft_logits, const int32_t* draft_lens,
                                const float* temperature, int B, int D, int V, float factor,
                                int k, hipStream_t stream) {
  return sv::saguaro_reshape(dtype, draft_logits, draft_lens, temperature, B, D, V, factor, k,
                             nullptr, 0, stream);
}

size_t spec_verify_saguaro_workspace_bytes(int B, int D, int V) {
  return sv::sag_workspace_bytes(B, D, V);
}

int spec_verify_saguaro_reshape_ws(int dtype, void* draft_logits, const int32_t* draft_lens,
                                   const float* temperature, int B, int D, int V, float factor,
                                   int k, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  if (workspace == nullptr) return SV_EINVAL;
  return sv::saguaro_reshape(dtype, draft_logits, draft_lens, temperature, B, D, V, factor, k,
                             workspace, workspace_bytes, stream);
}

int spec_verify_advance(const int32_t* accept_len, const int32_t* tokens, int B, int D,
                        int32_t* input_ids, int W, int32_t* seq_len, hipStream_t stream) {
  return sv::advance(accept_len, tokens, B, D, input_ids, W, seq_len, stream);
}

const char* spec_verify_strerror(int code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument";
    case SV_EDTYPE: return "unknown dtype";
    case SV_EHIP: return "HIP runtime error";
    case SV_ENODEV: return "no usable GPU device";
    case SV_ENOMEM: return "workspace allocation failed or workspace too small";
    case SV_ESCRATCH:
      return "problem needs more workspace than spec_verify_noalloc's fixed scratch holds";
    default: return "unknown status";
  }
}

int spec_verify_version(void) { return 303; }

int spec_verify_row_stages(int dtype, int B, int D, int V, int* cuts, int max_cuts) {
  if ((dtype != 0 && dtype != 1) || B <= 0 || D < 0 || D > SV_MAX_D || V <= 0 || !cuts)
    return SV_EINVAL;
  int c[sv::kMaxStages + 1];
  const int n = sv::stage_plan(true, B, D, V, dtype == 1 ? 2 : 4, c);
  for (int i = 0; i <= n && i < max_cuts; ++i) cuts[i] = c[i];
  return n;
}

int spec_verify_release(hipStream_t stream) {
  int dev = 0, count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return SV_ENODEV;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ENODEV;
  std::lock_guard<std::mutex> lock(sv::g_ws_mutex);
  int rc = SV_OK;
  for (auto* m : {&sv::g_ws, &sv::g_sag}) {
    auto it = m->find({dev, stream});
    if (it == m->end()) continue;
    if (it->second.ptr && hipFreeAsync(it->second.ptr, stream) != hipSuccess) rc = SV_EHIP;
    m->erase(it);
  }
  return rc;
}

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
