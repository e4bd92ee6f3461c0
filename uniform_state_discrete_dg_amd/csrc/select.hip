// select.hip -- the integer end of a denoising step: canvas initialisation,
// the entropy-bounded accept walk, re-noise and the adaptive-stop flags.
// One workgroup of 256 threads handles the whole canvas (N <= 256).
//
// [P3] §5.4: positions are ordered from lowest to highest entropy and walked
// in that order; a position is accepted while the running sum of entropies
// (less their maximum, which in ascending order is the current one) stays
// within the threshold, and the first failure ends the walk.  [P5] states
// the plain running sum (rule CUMSUM).  Every rejected position is
// re-noised with a fresh uniform token; accepted ones take the argmax.
//
// The walk is evaluated in parallel: keys (entropy bits << 32 | position)
// are bitonic-sorted, the entropies are turned into 2^-32-nat fixed point
// and prefix-summed in 64-bit integers, and rank r is accepted iff its
// prefix test holds -- the tests are monotone in r, so this equals the
// sequential walk, and integer sums make the result independent of order.
#include "dg_device.h"
#include "dg_kernels.h"
#include "dgdenoise.h"

namespace dg {

__global__ void canvas_init_kernel(int32_t *tokens, int32_t *status, int N, int log2v, uint64_t seed,
                                   uint32_t canvas_id) {
  const int i = threadIdx.x + blockIdx.x * blockDim.x;
  if (i < N) tokens[i] = uniform_token(seed, (uint32_t)i, 0u, canvas_id, 0u, log2v);
  if (i < DG_STATUS_WORDS) status[i] = (i == DG_ST_STEP) ? -1 : 0;
}

hipError_t canvas_init(int32_t *tokens, int32_t *status, int N, int log2v, uint64_t seed,
                       uint32_t canvas_id, hipStream_t s) {
  hipLaunchKernelGGL(canvas_init_kernel, dim3(1), dim3(256), 0, s, tokens, status, N, log2v, seed, canvas_id);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) select_kernel(const float *__restrict__ entropy,
                                                     const int32_t *__restrict__ argmax,
                                                     int32_t *__restrict__ tokens, uint8_t *__restrict__ accept,
                                                     int32_t *__restrict__ status, int N, int log2v,
                                                     uint64_t limit, int rule, float conf_eps, uint64_t seed,
                                                     uint32_t canvas_id, uint32_t step) {
  __shared__ uint64_t keys[256];
  __shared__ uint64_t scan[256];
  __shared__ uint8_t acc_pos[256];
  __shared__ float fmin_s[256], fmax_s[256], fsum_s[256];
  const int i = threadIdx.x;

  float h = 0.f;
  if (i < N) {
    h = entropy[i];
    if (h <= 0.f) h = 0.f;  // clamp; NaN passes through
  }
  keys[i] = (i < N) ? (((uint64_t)__float_as_uint(h) << 32) | (uint32_t)i) : ~0ull;
  acc_pos[i] = 0;
  __syncthreads();

  // bitonic sort, ascending
  for (int k = 2; k <= 256; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int ixj = i ^ j;
      if (ixj > i) {
        const uint64_t a = keys[i], b = keys[ixj];
        const bool up = (i & k) == 0;
        if ((a > b) == up) {
          keys[i] = b;
          keys[ixj] = a;
        }
      }
      __syncthreads();
    }
  }

  // fixed-point prefix sums over the sorted order (rank = i)
  const uint64_t key = keys[i];
  const bool real = key != ~0ull;
  const float hr = __uint_as_float((uint32_t)(key >> 32));
  const bool finite = real && (hr < 1048576.0f);  // NaN / inf / absurd end the walk
  const uint64_t q = finite ? (uint64_t)((double)hr * 4294967296.0) : 0ull;
  scan[i] = q;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const uint64_t v = (i >= o) ? scan[i - o] : 0ull;
    __syncthreads();
    scan[i] += v;
    __syncthreads();
  }
  const uint64_t incl = scan[i];
  const uint64_t test = (rule == DG_ACCEPT_CUMSUM) ? incl : incl - q;
  if (finite && test <= limit) acc_pos[(uint32_t)key] = 1;
  __syncthreads();

  // re-noise, new canvas, flags
  int changed = 0, conf = 1, acc = 0, isnan_ = 0;
  float hmin = INFINITY, hmax = -INFINITY, hsum = 0.f;
  if (i < N) {
    acc = acc_pos[i];
    const int32_t old = tokens[i];
    const int32_t t = acc ? argmax[i] : uniform_token(seed, (uint32_t)i, step, canvas_id, 1u, log2v);
    tokens[i] = t;
    accept[i] = (uint8_t)acc;
    changed = (t != old);
    conf = (h < conf_eps);  // false for NaN
    isnan_ = (h != h);
    hmin = fminf(hmin, h);
    hmax = fmaxf(hmax, h);
    hsum = isnan_ ? 0.f : h;
  }
  const int any_changed = __syncthreads_or(changed);
  const int all_conf = __syncthreads_and(conf);
  const int n_acc = __syncthreads_count(acc);
  const int n_nan = __syncthreads_count(isnan_);
  fmin_s[i] = hmin;
  fmax_s[i] = hmax;
  fsum_s[i] = hsum;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (i < o) {
      fmin_s[i] = fminf(fmin_s[i], fmin_s[i + o]);
      fmax_s[i] = fmaxf(fmax_s[i], fmax_s[i + o]);
      fsum_s[i] += fsum_s[i + o];
    }
    __syncthreads();
  }
  if (i == 0) {
    const int stable_old = status[DG_ST_STABLE];
    status[DG_ST_ALLCONF] = all_conf;
    status[DG_ST_CHANGED] = any_changed;
    status[DG_ST_STABLE] = any_changed ? 0 : stable_old + 1;
    status[DG_ST_ACCEPTED] = n_acc;
    status[DG_ST_NAN] = n_nan;
    status[DG_ST_STEP] = (int32_t)step;
    status[DG_ST_HMIN] = __float_as_int(fmin_s[0]);
    status[DG_ST_HMAX] = __float_as_int(fmax_s[0]);
    status[DG_ST_HMEAN] = __float_as_int(N > n_nan ? fsum_s[0] / (float)(N - n_nan) : 0.f);
  }
}

hipError_t select_step(const float *entropy, const int32_t *argmax, int32_t *tokens, uint8_t *accept,
                       int32_t *status, int N, int log2v, double gamma, int rule, float conf_eps,
                       uint64_t seed, uint32_t canvas_id, uint32_t step, hipStream_t s) {
  uint64_t limit = 0;
  if (gamma > 0.0) {
    const double x = gamma * 4294967296.0;
    limit = (x >= 18446744073709551615.0) ? ~0ull : (uint64_t)x;
  }
  hipLaunchKernelGGL(select_kernel, dim3(1), dim3(256), 0, s, entropy, argmax, tokens, accept, status, N,
                     log2v, limit, rule, conf_eps, seed, canvas_id, step);
  return hipGetLastError();
}

__global__ void philox_test_kernel(const uint32_t *ctr, uint32_t k0, uint32_t k1, uint32_t *out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const Philox4 o = philox4x32_10(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3], k0, k1);
  for (int k = 0; k < 4; ++k) out[4 * i + k] = o.v[k];
}

hipError_t philox_test(const uint32_t *ctr, uint32_t k0, uint32_t k1, uint32_t *out, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(philox_test_kernel, dim3((n + 255) / 256), dim3(256), 0, s, ctr, k0, k1, out, n);
  return hipGetLastError();
}

}  // namespace dg
