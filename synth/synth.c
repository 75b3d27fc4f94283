/*
 * Seeded synthetic decode-step inputs for the PPSA (position persistent sparse
 * attention) workloads.
 *
 * This module only manufactures inputs. It holds none of the attention or
 * selection arithmetic: it is shared by the float64 oracle (tests/bench CPU
 * leg) and by the HIP path (tests/bench GPU leg), which must see bit-identical
 * inputs.
 *
 * Randomness is counter based: every value is a pure function of
 * (seed, tensor tag, layer, batch, head, row, element), so any layer, batch
 * row or head can be regenerated on its own and threads never share state.
 *   - Hash: the SplitMix64 output function (Steele, Lea & Flood, "Fast
 *     splittable pseudorandom number generators", OOPSLA 2014), chained over
 *     the coordinates.
 *   - Normals: the Box-Muller transform on two 53-bit uniforms in (0, 1],
 *     evaluated in double and rounded once to float.
 *
 * Workload structure (heavy hitters): per KV head h a unit vector u_h is drawn
 * once and shared by every layer and batch row. Per (batch b, KV head h) a set
 * H_bh holds the sink positions 0..3 plus n_random positions drawn without
 * replacement from [4, N_b) by a partial Fisher-Yates shuffle; the set is the
 * same at every layer. Keys at positions in H_bh get +key_bias*u_h, every query
 * head of KV group h gets +q_bias*u_h, values are plain N(0,1). Biases are
 * added in float; bf16 outputs are rounded once, to nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TAG_Q 0x51ull
#define TAG_K 0x4Bull
#define TAG_V 0x56ull
#define TAG_U 0x55ull
#define TAG_HH 0x4848ull
#define TAG_LEN 0x4C454Eull

enum { PAD_ZERO = 0, PAD_NAN = 1, PAD_RANDOM = 2 };

static inline uint64_t sm_out(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Chain one more coordinate into a running key. */
static inline uint64_t sm_chain(uint64_t key, uint64_t coord) { return sm_out(key ^ sm_out(coord)); }

static uint64_t row_key(uint64_t seed, uint64_t tag, uint64_t layer, uint64_t b, uint64_t h, uint64_t n) {
  uint64_t k = sm_out(seed);
  k = sm_chain(k, tag);
  k = sm_chain(k, layer);
  k = sm_chain(k, b);
  k = sm_chain(k, h);
  k = sm_chain(k, n);
  return k;
}

/* Uniform in (0, 1] from the top 53 bits. */
static inline double unit_open0(uint64_t r) { return ((double)(r >> 11) + 1.0) * (1.0 / 9007199254740992.0); }

/* Two independent N(0,1) draws for element pair j of a row. */
static inline void normal_pair(uint64_t rkey, uint64_t j, double* z0, double* z1) {
  double u1 = unit_open0(sm_out(rkey + 2 * j));
  double u2 = unit_open0(sm_out(rkey + 2 * j + 1));
  double rad = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925 * u2;
  *z0 = rad * cos(th);
  *z1 = rad * sin(th);
}

/* Fill out[0..d) with the row's normals (d may be odd). */
static void normal_row(uint64_t rkey, int d, float* out) {
  for (int i = 0; i < d; i += 2) {
    double z0, z1;
    normal_pair(rkey, (uint64_t)(i / 2), &z0, &z1);
    out[i] = (float)z0;
    if (i + 1 < d) out[i + 1] = (float)z1;
  }
}

static inline uint16_t bf16_rne(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u); /* quiet NaN */
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

static inline void store_row(const float* src, int d, int out_bf16, void* dst, size_t row) {
  if (out_bf16) {
    uint16_t* o = (uint16_t*)dst + row * (size_t)d;
    for (int i = 0; i < d; ++i) o[i] = bf16_rne(src[i]);
  } else {
    memcpy((float*)dst + row * (size_t)d, src, sizeof(float) * (size_t)d);
  }
}

static inline void store_pad(int d, int out_bf16, int pad_mode, void* dst, size_t row) {
  if (out_bf16) {
    uint16_t v = pad_mode == PAD_NAN ? (uint16_t)0x7FC0u : (uint16_t)0u;
    uint16_t* o = (uint16_t*)dst + row * (size_t)d;
    for (int i = 0; i < d; ++i) o[i] = v;
  } else {
    float v = pad_mode == PAD_NAN ? NAN : 0.0f;
    float* o = (float*)dst + row * (size_t)d;
    for (int i = 0; i < d; ++i) o[i] = v;
  }
}

int synth_abi_version(void) { return 1; }

/* Ragged lengths: uniform integers in [nmin, nmax] (all nmax when equal). */
void synth_seq_lens(uint64_t seed, int batch, int nmin, int nmax, int32_t* out) {
  for (int b = 0; b < batch; ++b) {
    if (nmax <= nmin) {
      out[b] = nmax;
    } else {
      uint64_t r = row_key(seed, TAG_LEN, 0, (uint64_t)b, 0, 0);
      out[b] = nmin + (int32_t)(r % (uint64_t)(nmax - nmin + 1));
    }
  }
}

/* u[h] = z / |z| with z ~ N(0, I_d), one per KV head, layer independent. */
void synth_unit_vectors(uint64_t seed, int kv_heads, int d, float* u) {
  float* z = (float*)malloc(sizeof(float) * (size_t)d);
  for (int h = 0; h < kv_heads; ++h) {
    normal_row(row_key(seed, TAG_U, 0, 0, (uint64_t)h, 0), d, z);
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += (double)z[i] * (double)z[i];
    double inv = 1.0 / sqrt(s);
    for (int i = 0; i < d; ++i) u[(size_t)h * d + i] = (float)((double)z[i] * inv);
  }
  free(z);
}

/*
 * Heavy-hitter positions per (b, h): out is [batch, kv_heads, stride] with
 * stride >= 4 + n_random; count[b*kv_heads+h] says how many are used.
 * Returns 0, or -1 when stride is too small.
 */
int synth_heavy_positions(uint64_t seed, int batch, int kv_heads, const int32_t* seq_lens, int n_random,
                          int32_t* out, int32_t* count, int stride) {
  if (stride < 4 + (n_random > 0 ? n_random : 0)) return -1;
  int rc = 0;
#pragma omp parallel for schedule(dynamic)
  for (int bh = 0; bh < batch * kv_heads; ++bh) {
    int b = bh / kv_heads, h = bh % kv_heads;
    int n = seq_lens[b] > 0 ? seq_lens[b] : 0;
    int32_t* dst = out + (size_t)bh * stride;
    int c = 0;
    for (int s = 0; s < 4 && s < n; ++s) dst[c++] = s;
    int pool = n > 4 ? n - 4 : 0;
    int take = n_random < pool ? n_random : pool;
    if (take > 0) {
      int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)pool);
      if (!a) {
        rc = -2;
      } else {
        for (int i = 0; i < pool; ++i) a[i] = 4 + i;
        uint64_t key = row_key(seed, TAG_HH, 0, (uint64_t)b, (uint64_t)h, 0);
        for (int i = 0; i < take; ++i) {
          uint64_t r = sm_out(key + (uint64_t)i);
          int j = i + (int)(r % (uint64_t)(pool - i));
          int32_t t = a[i];
          a[i] = a[j];
          a[j] = t;
          dst[c++] = a[i];
        }
        free(a);
      }
    }
    count[bh] = c;
  }
  return rc;
}

/* q[b, hq, :] = N(0,1) + q_bias * u[hq / group], for one layer. */
void synth_fill_q(uint64_t seed, int layer, int batch, int q_heads, int kv_heads, int d, const float* u, float q_bias,
                  int out_bf16, void* out) {
  int group = q_heads / kv_heads;
#pragma omp parallel
  {
    float* row = (float*)malloc(sizeof(float) * (size_t)d);
#pragma omp for schedule(static)
    for (int bh = 0; bh < batch * q_heads; ++bh) {
      int b = bh / q_heads, hq = bh % q_heads;
      normal_row(row_key(seed, TAG_Q, (uint64_t)layer, (uint64_t)b, (uint64_t)hq, 0), d, row);
      const float* uh = u + (size_t)(hq / group) * d;
      for (int i = 0; i < d; ++i) row[i] = row[i] + q_bias * uh[i];
      store_row(row, d, out_bf16, out, (size_t)bh);
    }
    free(row);
  }
}

/*
 * K and V for one layer, [batch, kv_heads, max_len, d]. Rows at or past
 * seq_lens[b] are filled per pad_mode (zero, NaN, or the same draws as a live
 * row). heavy/heavy_count/stride come from synth_heavy_positions.
 */
void synth_fill_kv(uint64_t seed, int layer, int batch, int kv_heads, int max_len, int d, const int32_t* seq_lens,
                   const int32_t* heavy, const int32_t* heavy_count, int stride, const float* u, float key_bias,
                   int out_bf16, int pad_mode, void* k_out, void* v_out) {
  size_t pairs = (size_t)batch * (size_t)kv_heads;
  unsigned char* mark = (unsigned char*)calloc(pairs * (size_t)max_len, 1);
  for (size_t bh = 0; bh < pairs; ++bh)
    for (int i = 0; i < heavy_count[bh]; ++i) {
      int p = heavy[bh * (size_t)stride + i];
      if (p >= 0 && p < max_len) mark[bh * (size_t)max_len + p] = 1;
    }
  const int64_t chunk = 256;
  int64_t chunks_per_pair = ((int64_t)max_len + chunk - 1) / chunk;
  int64_t total = (int64_t)pairs * chunks_per_pair;
#pragma omp parallel
  {
    float* row = (float*)malloc(sizeof(float) * (size_t)d);
#pragma omp for schedule(dynamic, 4)
    for (int64_t t = 0; t < total; ++t) {
      size_t bh = (size_t)(t / chunks_per_pair);
      int b = (int)(bh / (size_t)kv_heads), h = (int)(bh % (size_t)kv_heads);
      int n0 = (int)((t % chunks_per_pair) * chunk);
      int n1 = n0 + (int)chunk < max_len ? n0 + (int)chunk : max_len;
      int live = seq_lens[b];
      const float* uh = u + (size_t)h * d;
      for (int n = n0; n < n1; ++n) {
        size_t r = bh * (size_t)max_len + (size_t)n;
        if (n >= live && pad_mode != PAD_RANDOM) {
          store_pad(d, out_bf16, pad_mode, k_out, r);
          store_pad(d, out_bf16, pad_mode, v_out, r);
          continue;
        }
        normal_row(row_key(seed, TAG_K, (uint64_t)layer, (uint64_t)b, (uint64_t)h, (uint64_t)n), d, row);
        if (mark[r])
          for (int i = 0; i < d; ++i) row[i] = row[i] + key_bias * uh[i];
        store_row(row, d, out_bf16, k_out, r);
        normal_row(row_key(seed, TAG_V, (uint64_t)layer, (uint64_t)b, (uint64_t)h, (uint64_t)n), d, row);
        store_row(row, d, out_bf16, v_out, r);
      }
    }
    free(row);
  }
  free(mark);
}

/* Round float to bf16 bits (nearest-even), for callers that build inputs by hand. */
void synth_round_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(in[i]);
}
