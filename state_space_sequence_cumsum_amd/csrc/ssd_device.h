// ssd_device.h -- gfx950 device helpers shared by the SSD kernels: element types,
// MFMA wrappers and the 32x32 accumulator lane layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// v_exp_f32: base-2 exponential on the transcendental unit.  Large positive
// arguments give +inf and large negative ones give 0, which is what the masked
// decay factors need.
__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// ---------------------------------------------------------------------------
// Element traits.  A "fragment" is the 8 values one lane contributes to one
// 32x32 MFMA tile for a 16-deep slice of the contraction index.  For bf16 that
// is one v_mfma_f32_32x32x16_bf16 operand.  For fp32 it is eight
// v_mfma_f32_32x32x2_f32 operands: in the e-th of those instructions lane l
// supplies element e, which the hardware places at contraction index l / 32.
// Because every operand of a product uses the same (lane, element) -> index
// assignment, any fixed assignment of the 16 logical indices to the pairs
// (l / 32, e) contracts correctly.
// ---------------------------------------------------------------------------
template <typename T> struct Elem;

template <> struct Elem<bf16> {
    typedef bf16x8 frag;
    typedef bf16x4 half;
    static __device__ __forceinline__ bf16 from_f32(float v) { return (bf16)v; }
};

template <> struct Elem<float> {
    typedef f32x8 frag;
    typedef f32x4 half;
    static __device__ __forceinline__ float from_f32(float v) { return v; }
};

__device__ __forceinline__ void mma(f32x16 &acc, const bf16x8 &a, const bf16x8 &b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x16 &acc, const f32x8 &a, const f32x8 &b)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
}

// Eight consecutive elements; p must be 16-byte aligned.
template <typename T> __device__ __forceinline__ typename Elem<T>::frag load_frag(const T *p);

template <> __device__ __forceinline__ bf16x8 load_frag<bf16>(const bf16 *p)
{
    return *reinterpret_cast<const bf16x8 *>(p);
}

template <> __device__ __forceinline__ f32x8 load_frag<float>(const float *p)
{
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4 *>(p + 4);
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f[e] = lo[e]; f[4 + e] = hi[e]; }
    return f;
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::frag zero_frag()
{
    typename Elem<T>::frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (T)0.0f;
    return f;
}

// 32x32 fp32 accumulator layout: element v of lane l holds row
// 8*(v/4) + 4*(l/32) + v%4 and column l%32.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

__device__ __forceinline__ f32x16 zero_acc()
{
    f32x16 a;
#pragma unroll
    for (int v = 0; v < 16; ++v) a[v] = 0.0f;
    return a;
}

// ---------------------------------------------------------------------------
// Raw buffer loads (MUBUF).  A resource covers `bytes` bytes from `base`; a load at
// a per-lane byte offset at or past the end returns zero (the hardware range check
// of a raw buffer, which sees the per-lane offset), so a tile that runs past the end
// of a sequence needs no clamping.  Word 3 is the gfx9 buffer configuration (32-bit
// data format, no swizzle).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes < 0 ? 0 : bytes,
                                             0x00020000);
}

__device__ __forceinline__ uint32_t buf_load_b32(rsrc_t r, uint32_t off)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

__device__ __forceinline__ u32x4 buf_load_b128(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Stores past the end of the range are dropped; with a zero-byte range the instructions
// still issue (and count in the wait counters) but write nothing.
__device__ __forceinline__ void buf_store_b32(rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}

__device__ __forceinline__ void buf_store_b128(rsrc_t r, uint32_t off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r,
                                           (int)off, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS transpose reads (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives, for e = 0..3, element i%4 of the 4-element row segment
// addressed by lane 4e + i/4 of the same group.  So if the 16 lanes address a
// 4 (k) x 16 (r) block of a k-major tile -- lane m pointing at row m/4, column
// 4*(m%4) -- lane i gets 4 consecutive k of column i: a k-packed MFMA operand
// read straight out of a tile stored in its natural (token-major) layout.
// ---------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ bf16x4 tr_read4(const bf16 *p)
{
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi)
{
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per-lane element offset of the transpose-read fragment of a k-major tile with
// row pitch `pitch` (elements).  Natural order: element e of lane l is row
// 8*(l/32) + e; column l%32.  The second 4-row read sits 4 rows further on.
__device__ __forceinline__ int tr_off_natural(int lane, int pitch)
{
    return (8 * (lane >> 5) + ((lane & 15) >> 2)) * pitch + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
}

// Accumulator order: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4, the row
// order in which a 32x32 accumulator hands its 16-deep half to a lane.  The
// second 4-row read sits 8 rows further on.
__device__ __forceinline__ int tr_off_accorder(int lane, int pitch)
{
    return (4 * (lane >> 5) + ((lane & 15) >> 2)) * pitch + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
}

// Row pitch (elements, bf16) for transpose-read tiles: at least `cols`, a
// multiple of 8 (16-byte rows), and an odd multiple of 32 bytes modulo 128 so
// that the four rows one 16-lane group touches fall in distinct bank ranges.
constexpr int tr_pitch(int cols)
{
    int b = (cols * 2 + 31) / 32 * 32;
    while ((b % 128) != 32 && (b % 128) != 96) b += 32;
    return b / 2;
}

// Row pitch (elements, bf16) for tiles read with 16-byte fragments (lane l: row
// l%32, bytes 16*(l/32) of a 32-byte k-slice): 16 bytes more than a multiple of
// 128 bytes so 16 consecutive rows hit 16 distinct 16-byte bank groups.
constexpr int frag_pitch(int cols)
{
    int b = (cols * 2 + 127) / 128 * 128 + 16;
    return b / 2;
}

// ---------------------------------------------------------------------------
// Register transposes for staging token-major global tiles into k-packed LDS
// rows (8 consecutive tokens of one column = one 16-byte MFMA fragment).
// ---------------------------------------------------------------------------
// Halves h of two dwords packed as (lo = a.h, hi = b.h).
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, int h)
{
    return __builtin_amdgcn_perm(b, a, h ? 0x07060302u : 0x05040100u);
}

// bf16 <-> fp32 on raw bits (bf16 is the upper half of an fp32)
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    bf16x2_t r;
    r[0] = (bf16)lo;
    r[1] = (bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------------------
// s_waitcnt immediate with vmcnt = n and expcnt, lgkmcnt at their maxima (gfx9 encoding)
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// f(std::integral_constant<int, i>) for i = 0 .. n - 1, unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// Wave-wide (64-lane) prefix sums on DPP lane moves, with no LDS round trip per step.
// The inclusive sum takes Hillis-Steele steps of 1, 2, 4 and 8 lanes within each row of
// 16 lanes, then carries the row totals across rows (broadcasts of lanes 15 and 31);
// a lane that receives nothing adds 0.  Every kernel that needs the same sums bit for bit
// (the stage-1 cumsum and the one-launch forward) uses this one order.
template <int CTRL, int ROW_MASK> __device__ __forceinline__ float dpp_move(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                  ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_inclusive_sum(float v)
{
    v += dpp_move<0x111, 0xf>(v);   // row_shr:1
    v += dpp_move<0x112, 0xf>(v);   // row_shr:2
    v += dpp_move<0x114, 0xf>(v);   // row_shr:4
    v += dpp_move<0x118, 0xf>(v);   // row_shr:8
    v += dpp_move<0x142, 0xa>(v);   // row_bcast:15, into rows 1 and 3
    v += dpp_move<0x143, 0xc>(v);   // row_bcast:31, into rows 2 and 3
    return v;
}
// lane l gets lane l-1's value, lane 0 gets 0 (wave_shr:1)
__device__ __forceinline__ float wave_shift_up1(float v) { return dpp_move<0x138, 0xf>(v); }
// lane `src` (the same for every lane of the wave)'s value
__device__ __forceinline__ float wave_read(float v, int src)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}

}  // namespace ssd
