/* gen.c -- seeded synthetic input generator (normal, Student-t, permutations) for the NVFP4
 * workloads.  It holds no part of the quantization method: only the random inputs that both the
 * HIP library and the CPU oracle are fed with.
 *
 * Random words: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
 * 1, 2, 3", SC 2011: ten rounds of two 32x32->64 multiplies by 0xD2511F53 and 0xCD9E8D57, key bumped
 * by 0x9E3779B9 and 0xBB67AE85 after each round), keyed by (low 32 bits of the seed, tensor id), with
 * counter (j low, j high, stream, 0x5EED5EED): word j/4 of call j gives the j-th 32-bit word of
 * stream `stream`.  The fourth counter word keeps these streams apart from any other user of
 * Philox keyed the same way.
 * Uniforms: u = (w + 0.5) / 2^32, in (0, 1).
 * Normals: Box-Muller in double; call c of a stream (four words u0..u3) gives normals 4c .. 4c + 3 =
 * r0 cos(2 pi u1), r0 sin(2 pi u1), r1 cos(2 pi u3), r1 sin(2 pi u3) with r = sqrt(-2 ln u0|u2).
 * A value times std is rounded to binary32 (round to nearest even), then, for bf16 outputs, to bf16
 * (round to nearest even on the bit pattern; finite values only).
 * Element i depends only on (seed, tensor id, stream, i), so the result does not depend on the
 * number of threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c[0] * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c[2] * 0xCD9E8D57u;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

static void words(uint64_t call, uint64_t seed, uint32_t tensor_id, uint32_t stream, uint32_t w[4]) {
  w[0] = (uint32_t)call;
  w[1] = (uint32_t)(call >> 32);
  w[2] = stream;
  w[3] = 0x5EED5EEDu;
  philox(w, (uint32_t)seed, tensor_id);
}

static double uniform(uint32_t w) { return ((double)w + 0.5) * 0x1p-32; }

/* normals 4 call .. 4 call + 3 of a stream */
static void normals4(uint64_t call, uint64_t seed, uint32_t tensor_id, uint32_t stream, double z[4]) {
  uint32_t w[4];
  words(call, seed, tensor_id, stream, w);
  const double two_pi = 6.283185307179586476925286766559;
  for (int p = 0; p < 2; ++p) {
    const double r = sqrt(-2.0 * log(uniform(w[2 * p])));
    const double t = two_pi * uniform(w[2 * p + 1]);
    z[2 * p] = r * cos(t);
    z[2 * p + 1] = r * sin(t);
  }
}

static uint16_t bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

/* kind 0: normal * scale; kind 1: Student-t(nu) * scale = z0 / sqrt(sum_{s=1..nu} z_s^2 / nu) with
 * z_s the element's normal of stream s */
typedef struct {
  void *out;
  int64_t begin, end;
  uint64_t seed;
  uint32_t tensor_id;
  double scale;
  int kind, nu, bf16;
} Job;

static void *run(void *arg) {
  const Job *j = (const Job *)arg;
  for (int64_t i = j->begin; i < j->end;) {
    const uint64_t call = (uint64_t)i >> 2;
    double v[4];
    normals4(call, j->seed, j->tensor_id, 0, v);
    if (j->kind == 1) {
      double chi[4] = {0, 0, 0, 0}, z[4];
      for (int s = 1; s <= j->nu; ++s) {
        normals4(call, j->seed, j->tensor_id, (uint32_t)s, z);
        for (int e = 0; e < 4; ++e) chi[e] += z[e] * z[e];
      }
      for (int e = 0; e < 4; ++e) v[e] = v[e] / sqrt(chi[e] / j->nu);
    }
    for (int e = (int)(i & 3); e < 4 && i < j->end; ++e, ++i) {
      const float f = (float)(v[e] * j->scale);
      if (j->bf16)
        ((uint16_t *)j->out)[i] = bf16_rne(f);
      else
        ((float *)j->out)[i] = f;
    }
  }
  return 0;
}

static void fill(void *out, int64_t n, uint64_t seed, uint32_t tensor_id, double scale, int kind, int nu,
                 int bf16, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  if (n < 4096) threads = 1;
  pthread_t th[64];
  Job jobs[64];
  const int64_t per = ((n + threads - 1) / threads + 3) & ~(int64_t)3;
  int started = 0;
  for (int t = 0; t < threads; ++t) {
    const int64_t b = t * per, e = b + per < n ? b + per : n;
    if (b >= e) break;
    jobs[t] = (Job){out, b, e, seed, tensor_id, scale, kind, nu, bf16};
    if (threads == 1 || pthread_create(&th[t], 0, run, &jobs[t]) != 0) {
      run(&jobs[t]);
      th[t] = 0;
    }
    ++started;
  }
  for (int t = 0; t < started; ++t)
    if (threads > 1 && th[t]) pthread_join(th[t], 0);
}

void sg_normal(void *out, int64_t n, uint64_t seed, uint32_t tensor_id, double stddev, int bf16, int threads) {
  fill(out, n, seed, tensor_id, stddev, 0, 0, bf16, threads);
}

void sg_student_t(void *out, int64_t n, int nu, double scale, uint64_t seed, uint32_t tensor_id, int bf16,
                  int threads) {
  fill(out, n, seed, tensor_id, scale, 1, nu, bf16, threads);
}

/* A uniformly drawn permutation of 0 .. n-1 (Fisher-Yates, Durstenfeld's order): for i = n-1 down to
 * 1, swap element i with element floor(w (i + 1) / 2^32), w the next word of the stream. */
void sg_permutation(int64_t *out, int64_t n, uint64_t seed, uint32_t tensor_id, uint32_t stream) {
  for (int64_t i = 0; i < n; ++i) out[i] = i;
  uint32_t w[4];
  uint64_t k = 0;
  for (int64_t i = n - 1; i >= 1; --i, ++k) {
    if ((k & 3) == 0) words(k >> 2, seed, tensor_id, stream, w);
    const int64_t j = (int64_t)(((uint64_t)w[k & 3] * (uint64_t)(i + 1)) >> 32);
    const int64_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/* the raw words of a stream (for the generator's own tests) */
void sg_words(uint32_t *out, int64_t ncalls, uint64_t seed, uint32_t tensor_id, uint32_t stream) {
  for (int64_t c = 0; c < ncalls; ++c) words((uint64_t)c, seed, tensor_id, stream, out + 4 * c);
}
