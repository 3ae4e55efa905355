// Device-side building blocks shared by the gfx950 kernels: vector types, the
// LDS tile layouts and their fragment reads, element conversions and the
// workgroup -> output-tile mapping.
//
// MFMA operand layout used throughout (measured on gfx950): for a 32x32xKb
// instruction with E elements per lane, lane l supplies row/column (l % 32) and
// the E consecutive k-values E*(l/32) .. E*(l/32)+E-1 of the block; result
// register r of lane l holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
// Kernels issue mfma(Bfrag, Afrag), so a lane's results are 4 consecutive
// output columns of one output row -- one 8-byte (bf16) or 4-byte (int8) store.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace omm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define OMM_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// ---------------------------------------------------------------------------
// LDS tile layouts.  Every operand tile holds BK k-values of BMN rows/columns.
//
// "K-major" tile (operand stored with k contiguous in memory): R rows (m or n)
// of 128 bytes of k (64 x 16-bit or 128 x 8-bit values) = 8 chunks of 16 bytes.
// Row r occupies bytes 128 r .. 128 r + 127 and its chunk c sits in slot
// c ^ kswz(r), kswz(r) = (r / 2) % 8.  A fragment read (ds_read_b128) puts 16
// consecutive lanes on 16 consecutive rows and one chunk; with the xor they
// cover the 16 slots of a 256-byte window (two rows): no bank conflicts with 64
// banks.  Any 8 consecutive rows are one 1 KiB block, which one DMA
// instruction fills from 8 whole 128-byte row segments.
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }
template <int R>
__device__ __forceinline__ int kmaj_off(int r, int c) {
    return (r << 7) + ((c ^ kswz(r)) << 4);
}
// per-lane part of a fragment read of chunk 2 s + l/32 at row block rb (a
// multiple of 32): kmaj_off(rb + l%32, 2 s + l/32) == rb*128 + kmaj_lane(l, s)
__device__ __forceinline__ int kmaj_lane(int lane, int s) {
    return ((lane & 31) << 7) + ((((2 * s) + (lane >> 5)) ^ kswz(lane & 31)) << 4);
}

// "MN-major" tile of 16-bit elements (operand stored with m or n contiguous):
// BK rows (k) of BMN elements.  32-byte granule g of row k is stored at
// granule g ^ mswz16(k), mswz16(k) = 2 (k % 4) + ((k / 4) ^ (k / 8)) % 2.
// Fragments are read with ds_read_b64_tr_b16, a 16-lane group covering 4
// consecutive rows (k = 4q .. 4q+3) of one granule: those 4 rows take 4
// distinct slots of one parity, so two groups on the same rows and adjacent
// granules (the 32x32x16 operand layout) or on the same granule and rows 8
// apart (the 16x16x32 layout) fill all 8 slots, i.e. every bank once per
// half-wave.  Measured on gfx950 the 32x32 pattern on such a swizzle gives the
// highest throughput of that instruction (~75 B/clk/CU against ~63 for a
// 4-row swizzle).
__device__ __forceinline__ int mswz16(int k) { return ((k & 3) << 1) + (((k >> 2) ^ (k >> 3)) & 1); }
template <int ROWB>
__device__ __forceinline__ int mmaj16_off(int k, int byte_in_row) {
    return k * ROWB + ((((byte_in_row >> 5) ^ mswz16(k))) << 5) + (byte_in_row & 31);
}

// "MN-major" tile of 8-bit elements: BK rows (k) of BMN bytes; 16-byte chunk c
// of row k is stored at chunk c ^ mswz8(k).  ds_read_b64_tr_b8 puts a 16-lane
// group on 8 consecutive rows of one chunk; mswz8 gives 8 distinct values mod 8
// and distinct halves (for chunk pairs c, c^1).
__device__ __forceinline__ int mswz8(int k) { return ((k & 7) << 1) + ((k >> 2) & 1); }
template <int ROWB>
__device__ __forceinline__ int mmaj8_off(int k, int byte_in_row) {
    return k * ROWB + ((((byte_in_row >> 4) ^ mswz8(k))) << 4) + (byte_in_row & 15);
}

// ---------------------------------------------------------------------------
// Conversions (round to nearest even).
// gfx950 converts fp32 to bf16 / fp16 in hardware (v_cvt_pk_bf16_f32,
// v_cvt_pk_f16_f32), rounding to nearest even under the default mode.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

template <int DT>  // 0 = bf16, 1 = fp16
__device__ __forceinline__ uint16_t to_bits(float f) {
    return DT == 0 ? f32_to_bf16_bits(f) : f32_to_f16_bits(f);
}
// two fp32 values -> one register of two 16-bit values (a in the low half)
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2_t v = {a, b};
    if constexpr (DT == 0)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
template <int DT>
__device__ __forceinline__ float from_bits(uint16_t b) {
    return DT == 0 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

template <int DT>
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
    if constexpr (DT == 0)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Workgroup -> tile mapping.  The dispatcher hands consecutive workgroup ids to
// the 8 XCDs round-robin; when the count divides by 8, id w is renumbered so
// that each XCD receives one contiguous run of the tile order (its own L2 then
// sees neighbouring tiles).  The run is walked in column strips GM tiles tall,
// so concurrently resident tiles share A row panels and B column panels.
__device__ __forceinline__ int xcd_remap(int w, int total) {
    if ((total & 7) == 0) return (w & 7) * (total >> 3) + (w >> 3);
    return w;
}
__device__ __forceinline__ void grouped_order(int w, int tiles_m, int tiles_n, int GM, int& tm, int& tn) {
    int per_group = GM * tiles_n;
    int g = w / per_group;
    int first = g * GM;
    int gm = min(tiles_m - first, GM);
    int r = w - g * per_group;
    tm = first + r % gm;
    tn = r / gm;
}

}  // namespace omm
