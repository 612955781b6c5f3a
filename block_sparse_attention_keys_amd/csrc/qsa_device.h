// Device helpers shared by the kernel sources (included inside
// `namespace qsa { namespace {`, so each translation unit has its own copy).
// gfx950: wave64, bf16 MFMA / dot2, buffer resources, DPP and row swaps.
#pragma once

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(4))) const uint32_t CU32;  // constant (scalar) memory

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return bf16_rne(x); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Buffer resource over [base, base + bytes): loads at or past the end return
// zeros (raw buffer, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// 16 bytes from lane src_byte / 4 (ds_bpermute: a lane permutation through
// the LDS crossbar, no LDS storage).
__device__ __forceinline__ uint4 lane_gather(uint4 v, int src_byte) {
  return make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.x),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.y),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.z),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.w));
}

constexpr uint32_t kOobOffset = 0xFFFFF000u;  // past the end of every buffer that uses it
constexpr int kStreamPolicy = 2;              // non-temporal: each K/V row is read once

// v combined with the value of lane l ^ 16 (or l ^ 32): the gfx950 row swaps
// hand each lane both values of its pair (in some order), on the VALU.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide reductions: four DPP steps inside each row of 16 lanes (xor 1,
// xor 2, half-row mirror, row mirror), then the two cross-row swaps.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp<0x140>(v));  // row_mirror
  return max_xor32(max_xor16(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return sum_xor32(sum_xor16(v));
}

// Wave-local ordering of LDS traffic (within one wave; the waves of a workgroup
// may be at different points).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Rotate-half RoPE of value x of a row held in LDS (the first R values
// rotate; the pair of x < R/2 is x + R/2).  freq: the frequency table
// (theta^(-2i/R), fp64; read with a direct index so that a kernel-argument
// table stays in the argument segment).  The angle pos * freq[i] is fp64, its
// cosine and sine are rounded to fp32, and the rotation is fp32 (products
// rounded, then the sum; the library is built without contraction).
__device__ __forceinline__ float rope_at(const float* row, int x, int R, const double* freq,
                                         int64_t pos) {
  if (x >= R) return row[x];
  const int h = R >> 1, i = x < h ? x : x - h;
  const double ang = (double)pos * freq[i];
  const float c = (float)cos(ang), sn = (float)sin(ang);
  if (x < h) return row[x] * c - row[x + h] * sn;
  return row[x] * c + row[i] * sn;
}

// ---------------------------------------------------------------------------
// Query positions and cache rows (every attention kernel resolves rows this way).

// Sequence of token t: the largest b with cu_q[b] <= t (cu_q ascending,
// cu_q[0] = 0).  The wave reads 64 offsets at a time and counts them with a
// ballot, so a batch of up to 64 sequences costs one memory round trip
// instead of a chain of log2(B) dependent loads.  Wave-uniform result.
__device__ __forceinline__ int seq_of(const int32_t* cu_q, int B, int t) {
  const int lane = threadIdx.x & 63;
  int count = 0;
  for (int b0 = 1; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const bool le = (b < B) && (cu_q[b] <= t);
    const int c = __popcll(__ballot(le));
    count += c;
    if (c < 64) break;
  }
  return count;
}

struct QueryPos {
  int b, p;
  bool ok;
};
// With one new token per sequence, token t is sequence t's token and cu_q[t]
// = t: one load instead of three dependent ones.
__device__ __forceinline__ QueryPos query_pos(const Geo& g, int t) {
  QueryPos q;
  if (g.one_q) {
    q.b = t;
    q.p = g.past_len[t];
  } else {
    q.b = seq_of(g.cu_q, g.B, t);
    q.p = g.past_len[q.b] + (t - g.cu_q[q.b]);
  }
  q.ok = q.p >= 0 && q.p < g.cap;
  return q;
}

// Element offset of row s of (sequence b, KV head kvh) in a K or V cache, or -1
// when the row is outside the stated capacity / page pool.
__device__ __forceinline__ int64_t kv_row(const Geo& g, int b, int kvh, int s) {
  if (s < 0 || s >= g.cap) return -1;
  if (g.page_table == nullptr) return ((int64_t)(b * g.Hkv + kvh) * g.cap + s) * g.D;
  const int page = g.page_table[(int64_t)b * g.max_pages + (s >> g.log2ps)];
  if (page < 0 || page >= g.n_pages) return -1;
  return (((int64_t)page * g.Hkv + kvh) * g.page_size + (s & (g.page_size - 1))) * g.D;
}

// ---------------------------------------------------------------------------
// 8-bit K/V in the Sylvester-Hadamard basis.

// Walsh-Hadamard butterfly stage across lanes for elements spread over
// lanes: the partner element sits `dl` lanes away; the element whose index
// has the stage bit set takes (partner - own), the other (own + partner), as
// in the in-place transform (x[j], x[j+len]) <- (x[j] + x[j+len], x[j] - x[j+len]).
__device__ __forceinline__ float fwht_cross(float v, int dl, bool upper) {
  const float o = __shfl_xor(v, dl, 64);
  return upper ? (o - v) : (v + o);
}

// The attention output of one head (D = 128) spread EPT consecutive dims per
// thread over 128/EPT consecutive lanes of a wave (t_in: the thread's rank
// among them): with the rotated basis, o = H o' (the 1/D is in out_scale),
// then the 8-bit storage's output scale.  All lanes of the wave take part.
template <int EPT>
__device__ __forceinline__ void kv8_output(const Geo& g, float (&o)[EPT], int t_in) {
  if (g.rot) {
#pragma unroll
    for (int len = 1; len < EPT; len <<= 1)
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if (!(i & len)) {
          const float a = o[i], b = o[i + len];
          o[i] = a + b;
          o[i + len] = a - b;
        }
#pragma unroll
    for (int dl = 1; dl * EPT < 128; dl <<= 1)
#pragma unroll
      for (int i = 0; i < EPT; ++i) o[i] = fwht_cross(o[i], dl, (t_in & dl) != 0);
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) o[i] *= g.out_scale;
}
