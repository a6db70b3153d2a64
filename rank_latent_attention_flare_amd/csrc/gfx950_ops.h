// Device helpers shared by the gfx950 kernel files: MFMA and operand types,
// lane-pair reductions, the swizzled LDS row layout, the encode's token order
// and transposed LDS reads. Included inside namespace flare { namespace { }.
#pragma once

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum / max of a value over the lane pair (l, l^32), same result in both lanes.
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Wait until at most N vector memory operations of this wave are outstanding
// (they complete in issue order); LDS and scalar counters are left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }
__device__ __forceinline__ bool wave_all(bool p) { return __ballot(!p) == 0; }

// Byte offset of 16-byte chunk `ch` of row `row` in an LDS tile of bf16 rows
// of width D. Chunks are XOR-swizzled per row so that the row-strided reads
// of the MFMA operands spread over the banks.
template <int D>
__device__ __forceinline__ int tile_off(int row, int ch) {
    constexpr int CH = D / 8;
    constexpr int ROWS_PER_256B = (256 / (2 * D)) > 0 ? (256 / (2 * D)) : 1;
    const int sw = (row / ROWS_PER_256B) & (CH - 1);
    return row * (2 * D) + ((ch ^ sw) << 4);
}

// Token (0..31) held by MFMA row r of the encode's S^T = K Q^T product. The
// order makes accumulator registers 8j..8j+7 of a lane hold 8 consecutive
// tokens, i.e. exactly the k-slots the P.V product needs as its B operand.
__device__ __forceinline__ int enc_row_token(int r) {
    const int grp = r >> 3, hi = (r >> 2) & 1, lo = r & 3;
    return ((grp >> 1) << 4) + (hi << 3) + ((grp & 1) << 2) + lo;
}

__device__ __forceinline__ bf16x8 zero8() {
    u32x4 z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8, z);
}

// Transposed LDS reads (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i%4 of the 64-bit words of lanes 4k + i/4 of the group.
// Two reads form one 8 x bf16 MFMA operand; lds_tr_op2 reads two operands.
// It is inline asm that waits for its own results before returning: with the
// compiler builtin, the compiler drains every outstanding global->LDS
// transfer (vmcnt(0)) before the read, which would empty the prefetch ring on
// every sub-block. Callers order these reads after the transfers they need
// (explicit vmcnt wait, then barrier).
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}
__device__ __forceinline__ void lds_tr_op2(const unsigned char* p1, const unsigned char* p2,
                                           const unsigned char* p3, const unsigned char* p4, bf16x8& o1,
                                           bf16x8& o2) {
    u32x2 w1, w2, w3, w4;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w1), "=&v"(w2), "=&v"(w3), "=&v"(w4)
        : "v"(lds_addr(p1)), "v"(lds_addr(p2)), "v"(lds_addr(p3)), "v"(lds_addr(p4))
        : "memory");
    const u32x4 a = {w1[0], w1[1], w2[0], w2[1]};
    const u32x4 b = {w3[0], w3[1], w4[0], w4[1]};
    o1 = __builtin_bit_cast(bf16x8, a);
    o2 = __builtin_bit_cast(bf16x8, b);
}

// The same reads through the compiler builtin, for kernels that move no data
// by global->LDS transfers: the compiler then places the waits itself and can
// keep several of these reads in flight.
__device__ __forceinline__ void lds_tr_op2_c(const unsigned char* p1, const unsigned char* p2,
                                             const unsigned char* p3, const unsigned char* p4, bf16x8& o1,
                                             bf16x8& o2) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    auto rd = [](const unsigned char* p) {
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                             (lds_s16x4*)(const __attribute__((address_space(3))) unsigned char*)p));
    };
    const u32x2 w1 = rd(p1), w2 = rd(p2), w3 = rd(p3), w4 = rd(p4);
    const u32x4 a = {w1[0], w1[1], w2[0], w2[1]};
    const u32x4 b = {w3[0], w3[1], w4[0], w4[1]};
    o1 = __builtin_bit_cast(bf16x8, a);
    o2 = __builtin_bit_cast(bf16x8, b);
}

