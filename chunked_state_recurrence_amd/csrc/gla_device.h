// gla_device.h — device helpers shared by the forward and backward kernels of
// libgla.so: element types and MFMA fragments, buffer descriptors, direct-to-
// LDS loads, explicit waits, LDS barriers, raw row loads, wave shapes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSpanGuard = 80.0f;  // log2 units: factors stay within 2^+-80

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Element types.  bf16: one v_mfma_f32_16x16x32_bf16 per 32-deep step.  f32:
// the same 32-deep step as eight v_mfma_f32_16x16x4f32.  Both take operand
// fragments of 8 values per lane: lane l holds row/column (l & 15) and the 8
// reduction positions {8*(l>>4) .. +7} of a 32-deep block.  Any fixed
// assignment of reduction positions works as long as both operands use it.
// ---------------------------------------------------------------------------
struct BF16 {
    using gmem_t = uint16_t;
    using lds_t = __bf16;
    using frag_t = bf16x8_t;
    __device__ static float g2f(gmem_t x) { return __uint_as_float(uint32_t(x) << 16); }
    __device__ static lds_t f2l(float x) { return (__bf16)x; }
    __device__ static float l2f(lds_t x) { return (float)x; }
    __device__ static frag_t ld_frag(const lds_t *p) { return *reinterpret_cast<const frag_t *>(p); }
    __device__ static void st_frag(lds_t *p, frag_t f) { *reinterpret_cast<frag_t *>(p) = f; }
    __device__ static frag_t pack(const float *x) {
        frag_t f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (__bf16)x[i];
        return f;
    }
    __device__ static void unpack(frag_t f, float *x) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)f[i];
    }
    __device__ static f32x4_t mma(frag_t a, frag_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // Row r of a padded row-major bf16 tile of pitch `pitch` bytes starts at
    // r * pitch + 128 * (r / 8): with pitch = 32 mod 256 the four rows one
    // transposing read touches cover distinct banks, and the extra shift puts
    // rows eight apart (the next 16-lane group) on the other half of the banks.
    __device__ static int rowoff(int r, int pitch) { return r * pitch + 128 * (r >> 3); }
    static constexpr int tile_bytes(int rows, int pitch) { return rows * pitch + 128 * (rows / 8); }
    // 8 consecutive tokens of one column from such a tile, k0 a multiple of 8:
    // two transposing reads of 4 tokens each.  Within each 16-lane group,
    // lane j supplies row k0 + j/4, columns c0 + 4(j%4)..+3 and receives
    // column c0 + (its index) of rows k0..k0+3.
    __device__ static frag_t ld_col8(const unsigned char *tile, int pitch, int k0, int c0, int n16) {
        typedef short s4_t __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s4_t *lds_s4_p;
        const unsigned char *a = tile + rowoff(k0, pitch) + (n16 >> 2) * pitch + (c0 + 4 * (n16 & 3)) * 2;
        const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_p)(a));
        const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_p)(a + 4 * pitch));
        typedef short s8_t __attribute__((ext_vector_type(8)));
        const s8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(frag_t, v);
    }
    // the same from two runs of 4 rows, k_lo.. and k_hi..: the order in which
    // a 16 x 16 accumulator pair (rows 4 q4 + e of tiles 2 ts and 2 ts + 1)
    // holds a 32-deep token step, so such a pair packed to bf16 is the other
    // operand as it stands
    __device__ static frag_t ld_col4x2(const unsigned char *tile, int pitch, int k_lo, int k_hi, int c0, int n16) {
        typedef short s4_t __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s4_t *lds_s4_p;
        const int lane_off = (n16 >> 2) * pitch + (c0 + 4 * (n16 & 3)) * 2;
        const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_p)(tile + rowoff(k_lo, pitch) + lane_off));
        const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_p)(tile + rowoff(k_hi, pitch) + lane_off));
        typedef short s8_t __attribute__((ext_vector_type(8)));
        const s8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(frag_t, v);
    }
    // store 4 consecutive outputs (8 bytes) at byte offset `off`
    __device__ static void st4(__amdgpu_buffer_rsrc_t r, int off, f32x4_t v) {
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        typedef unsigned int u2_t __attribute__((ext_vector_type(2)));
        bf16x4_t b;
        b[0] = (__bf16)v[0]; b[1] = (__bf16)v[1]; b[2] = (__bf16)v[2]; b[3] = (__bf16)v[3];
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2_t, b), r, off, 0, 0);
    }
};

struct F32 {
    using gmem_t = float;
    using lds_t = float;
    using frag_t = f32x8_t;
    __device__ static float g2f(gmem_t x) { return x; }
    __device__ static lds_t f2l(float x) { return x; }
    __device__ static float l2f(lds_t x) { return x; }
    __device__ static frag_t ld_frag(const lds_t *p) {
        const f32x4_t a = reinterpret_cast<const f32x4_t *>(p)[0];
        const f32x4_t b = reinterpret_cast<const f32x4_t *>(p)[1];
        frag_t f;
        f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
        f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
        return f;
    }
    __device__ static void st_frag(lds_t *p, frag_t f) {
        reinterpret_cast<f32x4_t *>(p)[0] = f32x4_t{f[0], f[1], f[2], f[3]};
        reinterpret_cast<f32x4_t *>(p)[1] = f32x4_t{f[4], f[5], f[6], f[7]};
    }
    __device__ static frag_t pack(const float *x) {
        frag_t f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = x[i];
        return f;
    }
    __device__ static void unpack(frag_t f, float *x) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = f[i];
    }
    __device__ static f32x4_t mma(frag_t a, frag_t b, f32x4_t c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
        return c;
    }
    // dense rows (fp32 tiles are loaded 1 KB at a time)
    __device__ static int rowoff(int r, int pitch) { return r * pitch; }
    static constexpr int tile_bytes(int rows, int pitch) { return rows * pitch; }
    __device__ static frag_t ld_col8(const unsigned char *tile, int pitch, int k0, int c0, int n16) {
        const float *a = reinterpret_cast<const float *>(tile + k0 * pitch) + c0 + n16;
        frag_t f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = a[e * (pitch / 4)];
        return f;
    }
    __device__ static void st4(__amdgpu_buffer_rsrc_t r, int off, f32x4_t v) {
        typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, v), r, off, 0, 0);
    }
};

// Buffer descriptors (gfx9 raw buffers): a load past num_records returns 0
// and a store past it is dropped, which masks the partial last chunk
// without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, long bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, int(bytes), 0x00020000);
}

// Buffer loads that write LDS directly: lane l's `size` bytes land at
// lds + l * size (lds must be uniform).  Loads past num_records write zeros.
typedef __attribute__((address_space(3))) void *lds_ptr_t;
template <int SIZE>
__device__ __forceinline__ void dma(rsrc_t r, void *lds, int voff, int soff) {
    static_assert(SIZE == 4 || SIZE == 16, "direct load size");
    if constexpr (SIZE == 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds), 4, voff, soff, 0, 0);
    if constexpr (SIZE == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds), 16, voff, soff, 0, 0);
}
// The same direct-to-LDS load issued from inline assembly.  The compiler's
// wait insertion then does not know about it: it adds no wait before later
// LDS reads or writes for it (it cannot tell which of them alias the load's
// target, so for the builtin form it waits for every such load in flight,
// which stalls a prefetch at the next LDS access).  Every consumer must wait
// for it explicitly (wait_vmem, then a barrier where other waves read it).
// The descriptor is passed as its four words (see rsrc_words), the LDS
// destination as a byte address (lds_addr): lane l's SIZE bytes land at
// lds + l * SIZE.  The leading s_nop covers the wait states a VMEM read of an
// SGPR just written by a VALU instruction needs, the second one those of a
// direct load after an M0 write.
__device__ __forceinline__ u32x4_t rsrc_words(const void *base, long bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return u32x4_t{uint32_t(a), uint32_t(a >> 32) & 0xffffu, uint32_t(bytes), 0x00020000u};
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)(p)));
}
// SALU_OPERANDS = true is for call sites whose SGPR operands are all written
// by scalar instructions (checked in the generated code): the leading s_nop is
// then left out.
template <int SIZE, bool SALU_OPERANDS = false>
__device__ __forceinline__ void dma_untracked(u32x4_t rs, uint32_t lds, int voff, int soff) {
    static_assert(SIZE == 4 || SIZE == 16, "direct load size");
    if constexpr (SALU_OPERANDS) {
        if constexpr (SIZE == 16)
            __asm__ __volatile__("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                                 :: "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
        else
            __asm__ __volatile__("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                                 :: "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
    } else {
        if constexpr (SIZE == 16)
            __asm__ __volatile__("s_nop 4\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                                 :: "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
        else
            __asm__ __volatile__("s_nop 4\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                                 :: "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
    }
}

// Wait until at most n vector-memory operations of this wave are in flight
// (operations retire in issue order).  The direct-to-LDS loads have no
// register results, so the compiler inserts no wait for them by itself.
// Counts above the counter's range (63) clamp down, which only waits longer.
template <int N0>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N0 >= 0, "vmcnt range");
    constexpr int N = N0 < 63 ? N0 : 63;
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Keeps the compiler from moving memory operations across this point, so
// the issue order the waits count on is the program order.
__device__ __forceinline__ void mem_fence_compiler() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Work-group barrier for LDS traffic: this wave's LDS reads and writes are
// complete, then every wave meets.  Unlike __syncthreads() it does not drain
// the wave's in-flight global loads (the release fence there counts the
// direct-to-LDS loads as pending LDS writes); those are waited for
// explicitly, with wait_vmem, before the barrier that publishes them.
__device__ __forceinline__ void block_sync() {
    __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// CPL consecutive elements of one row of q, k or v, as loaded from HBM.
template <typename E, int CPL> struct Raw;
template <> struct Raw<BF16, 2> {
    uint32_t x;
    __device__ void load(rsrc_t r, int off, int soff) { x = __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0); }
    __device__ float get(int u) const { return __uint_as_float(u ? (x & 0xffff0000u) : (x << 16)); }
    // column u of 8 consecutive rows, as a bf16 fragment (byte permutes, no conversion)
    __device__ static bf16x8_t col8(const Raw *r, int u) {
        u32x4_t w;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = __builtin_amdgcn_perm(r[2 * j + 1].x, r[2 * j].x, u ? 0x07060302u : 0x05040100u);
        return __builtin_bit_cast(bf16x8_t, w);
    }
};
template <> struct Raw<BF16, 1> {
    uint16_t x;
    __device__ void load(rsrc_t r, int off, int soff) { x = __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0); }
    __device__ float get(int) const { return __uint_as_float(uint32_t(x) << 16); }
    __device__ static bf16x8_t col8(const Raw *r, int) {
        u32x4_t w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = uint32_t(r[2 * j].x) | (uint32_t(r[2 * j + 1].x) << 16);
        return __builtin_bit_cast(bf16x8_t, w);
    }
};
template <> struct Raw<F32, 2> {
    u32x2_t x;
    __device__ void load(rsrc_t r, int off, int soff) { x = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0); }
    __device__ float get(int u) const { return __uint_as_float(u ? x.y : x.x); }
    __device__ static f32x8_t col8(const Raw *r, int u) {
        f32x8_t f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = r[j].get(u);
        return f;
    }
};
template <> struct Raw<F32, 1> {
    uint32_t x;
    __device__ void load(rsrc_t r, int off, int soff) { x = __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0); }
    __device__ float get(int) const { return __uint_as_float(x); }
    __device__ static f32x8_t col8(const Raw *r, int) {
        f32x8_t f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = r[j].get(0);
        return f;
    }
};
template <int CPL> struct RawG;
// Scalar gates (one per token) use the same registers: load_one / fill put
// the token's gate in every column slot.
template <> struct RawG<2> {
    u32x2_t x;
    __device__ void load(rsrc_t r, int off, int soff) { x = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0); }
    __device__ void load_one(rsrc_t r, int off, int soff) {
        const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
        x = u32x2_t{u, u};
    }
    __device__ void fill(float f) { x = u32x2_t{__float_as_uint(f), __float_as_uint(f)}; }
    __device__ float get(int u) const { return __uint_as_float(u ? x.y : x.x); }
};
template <> struct RawG<1> {
    uint32_t x;
    __device__ void load(rsrc_t r, int off, int soff) { x = __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0); }
    __device__ void load_one(rsrc_t r, int off, int soff) { load(r, off, soff); }
    __device__ void fill(float f) { x = __float_as_uint(f); }
    __device__ float get(int) const { return __uint_as_float(x); }
};

// Column position inside a row of the row-major q/k tiles in LDS.  Within
// every 32-column block, key dims {4a..4a+3} (a < 4) go to 8a.., and
// {16+4a..} go to 8a+4..: a fragment read of 8 consecutive positions then
// holds exactly the key dims of two 16-row accumulator tiles of S, so S can be
// fed to the MFMA straight from its accumulators.
__device__ __forceinline__ int perm_col(int c) {
    const int blk = c & ~31, in = c & 31, a = in >> 2, e = in & 3;
    return blk + (a < 4 ? (a << 3) + e : ((a - 4) << 3) + 4 + e);
}

// Waves per work-group: 8 chunk rows per wave while every wave still owns at
// least one 16-wide tile of value columns, else 16 rows per wave.
template <int D, int C> struct Shape {
    static constexpr int NW = (C / 8 < D / 16) ? C / 8 : D / 16;
    static constexpr int RPW = C / NW;   // chunk rows per wave (8, 16 or 32)
    static_assert(RPW == 8 || RPW == 16 || RPW == 32, "unsupported chunk / head-dim pair");
};

// The backward's bf16 chunk-start states: D x D in 16 x 16 tiles, tile
// (r / 16, c / 16) row-major over the tiles, each tile row-major (256
// elements); element offset of (r, c)
template <int D>
__device__ __forceinline__ int bf16_state_offset(int r, int c) {
    return ((r >> 4) * (D / 16) + (c >> 4)) * 256 + (r & 15) * 16 + (c & 15);
}

// 4 x 4 transpose across the lanes of a quad: lane j (= lane & 3) holds
// x[e] = M[j][e] on entry and x[e] = M[e][j] on exit.  Two exchanges: the
// off-diagonal 2 x 2 blocks with lane j ^ 2, then the off-diagonal entries of
// each 2 x 2 block with lane j ^ 1 (DPP quad permutes).
__device__ __forceinline__ void quad_transpose4(float (&x)[4], int j) {
    auto qp = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
    };
    const bool lo2 = (j & 2) == 0, lo1 = (j & 1) == 0;
    float s0 = lo2 ? x[2] : x[0], s1 = lo2 ? x[3] : x[1];
    float r0 = qp(s0, std::integral_constant<int, 0x4E>{}), r1 = qp(s1, std::integral_constant<int, 0x4E>{});   // lane j ^ 2
    if (lo2) { x[2] = r0; x[3] = r1; } else { x[0] = r0; x[1] = r1; }
    s0 = lo1 ? x[1] : x[0];
    s1 = lo1 ? x[3] : x[2];
    r0 = qp(s0, std::integral_constant<int, 0xB1>{});   // lane j ^ 1
    r1 = qp(s1, std::integral_constant<int, 0xB1>{});
    if (lo1) { x[1] = r0; x[3] = r1; } else { x[0] = r0; x[2] = r1; }
}

// N consecutive elements of an LDS row from fp32 with one store (N = 2 or 4;
// dst aligned to the store's size), element-wise for N = 1.  bf16 values are
// rounded to nearest even, one conversion per pair.
template <typename E, int N>
__device__ __forceinline__ void st_lds_cols(typename E::lds_t *dst, const float (&v)[N]) {
    using l_t = typename E::lds_t;
    if constexpr (N == 2 || N == 4) {
        typedef float fN_t __attribute__((ext_vector_type(N)));
        typedef l_t lN_t __attribute__((ext_vector_type(N)));
        fN_t x;
#pragma unroll
        for (int n = 0; n < N; ++n) x[n] = v[n];
        *reinterpret_cast<lN_t *>(dst) = __builtin_convertvector(x, lN_t);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) dst[n] = E::f2l(v[n]);
    }
}

// two floats as packed bf16 (round to nearest even), the first in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const __bf16 ha = (__bf16)a, hb = (__bf16)b;
    return uint32_t(__builtin_bit_cast(uint16_t, ha)) | (uint32_t(__builtin_bit_cast(uint16_t, hb)) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

}  // namespace gla
