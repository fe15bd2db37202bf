// mxfa_device.h -- gfx950 device helpers: vector types, bf16 packing, MFMA
// wrappers, exp2 and the mask / softcap transforms shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxfa_internal.h"

namespace mxfa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = kXcdCount;  // MI355X: 8 accelerator complex dies, each with its own L2

#define MXFA_DEV __device__ __forceinline__

// ---------------------------------------------------------------- conversions

// Two fp32 -> packed bf16x2 (round to nearest even; v_cvt_pk_bf16_f32).
MXFA_DEV uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t f = {lo, hi};
    bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

MXFA_DEV float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// acc + lo + hi of a packed bf16 pair, in one instruction (v_dot2c_f32_bf16
// against (1, 1): the products are exact, the sum is an fp32 add).
MXFA_DEV float add_bf16x2(uint32_t pair, float acc) {
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), ones, acc, false);
}

// ---------------------------------------------------------------- math

// 2^x on the hardware transcendental unit (v_exp_f32); exp2(-inf) = 0.
MXFA_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

MXFA_DEV float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

MXFA_DEV float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Raw score s (= <q, k>) -> logit in log2 units (score * log2 e), with the
// optional softcap applied to the scaled score:
//   no cap: x = s * scale * log2e
//   cap c : x = c * log2e * tanh(s * scale / c), tanh(y) = 1 - 2 / (exp(2y) + 1)
template <bool kCap>
MXFA_DEV float score_to_logit(float s, float x_mul, float cap_mul, float cap_out) {
    if constexpr (kCap) {
        const float e = fast_exp2(s * cap_mul);
        return cap_out - 2.0f * cap_out * fast_rcp(e + 1.0f);
    } else {
        return s * x_mul;
    }
}

// ---------------------------------------------------------------- visibility

// Key j is visible to the query at key position pos (bottom-right aligned)
// iff 0 <= j < sk, j <= pos (causal), pos - wl <= j (wl >= 0), j <= pos + wr (wr >= 0).
struct KeyRange {
    int lo;  // first visible key (inclusive)
    int hi;  // last visible key (inclusive); hi < lo: no key
};

MXFA_DEV KeyRange visible_range(int pos, int sk, int causal, int wl, int wr) {
    KeyRange r;
    r.lo = 0;
    r.hi = sk - 1;
    if (causal) r.hi = min(r.hi, pos);
    if (wr >= 0) r.hi = min(r.hi, pos + wr);
    if (wl >= 0) r.lo = max(r.lo, pos - wl);
    return r;
}

// ---------------------------------------------------------------- MFMA

// D = A * B + C for a 32x32 tile with a 16-deep contraction, bf16 inputs,
// fp32 accumulate. Lane l holds A row (l % 32) and B column (l % 32), eight
// contraction elements each (the same eight for A and B); D in the 32x32
// accumulator layout: lane l, register r -> column l % 32,
// row 8 * (r / 4) + 4 * (l / 32) + r % 4.
MXFA_DEV f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A * B + C for a 16x16 tile with a 32-deep contraction, bf16 inputs,
// fp32 accumulate. Lane l holds A row (l % 16) and B column (l % 16), eight
// contraction elements each (the same eight for A and B); D: lane l,
// register r -> column l % 16, row 4 * (l / 16) + r.
MXFA_DEV f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- memory

MXFA_DEV u32x4_t load_u32x4(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
MXFA_DEV void store_u32x4(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
MXFA_DEV void store_u32x2(void* p, u32x2_t v) { *reinterpret_cast<u32x2_t*>(p) = v; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

MXFA_DEV lds_ptr_t to_lds(void* p) { return (lds_ptr_t)p; }

// Buffer resource over [base, base + bytes): loads past the end return zero.
// Word 3 = 0x00020000: raw (untyped) 32-bit data, the gfx9 setting.
MXFA_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes lds_wave_base + 16 * l (the LDS base must be wave uniform).
MXFA_DEV void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t voffset,
                                uint32_t soffset = 0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, to_lds(lds_wave_base), 16, (int)voffset, (int)soffset, 0, 0);
}

// 16 bytes per lane from global memory into registers through a buffer
// resource (reads past the resource's end return zero).
MXFA_DEV u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voffset, (int)soffset, 0));
}

// Wait until this wave's outstanding vector-memory operations (including the
// LDS-bound buffer loads) have completed.
MXFA_DEV void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group, lane
// i supplies the address of 4 consecutive 16-bit elements; lane j receives
// element j % 4 of lanes 4e + j / 4 for e = 0..3. With lane i pointing at row
// i / 4, columns 4 * (i % 4) .. +3 of a 4 x 16 block, lane j gets column j of
// rows 0..3.
MXFA_DEV u32x2_t lds_read_tr16(const void* p) {
    bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

// Work-group barrier that orders LDS traffic only: this wave's LDS accesses
// complete, then s_barrier. Unlike __syncthreads() it does not wait for
// outstanding global loads (e.g. the next tile streaming into LDS).
MXFA_DEV void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

MXFA_DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr_t)(p); }

// Batches of transposing LDS reads issued from one asm block that also waits
// for them (lgkmcnt(0)) before it ends, so no read is in flight when the
// compiler takes the output registers over. Written in asm because the
// compiler treats the intrinsic as possibly aliasing in-flight LDS-bound
// buffer loads and would wait for those first. OFF is a byte offset added to
// every address (ds immediate offset).
template <int OFF>
MXFA_DEV void lds_read_tr16_x4(u32x2_t (&r)[4], const uint32_t (&a)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
        "ds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
        "ds_read_b64_tr_b16 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
        : "memory");
}

template <int OFF>
MXFA_DEV void lds_read_tr16_x8(u32x2_t (&r)[8], const uint32_t (&a)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF)
        : "memory");
}

// 16-byte LDS read at a byte address (ds_read_b128).
// Sixteen transposing reads: address a[i] at offsets OFF0, OFF1, OFF2, OFF3
// for i = 0..3 (read 4*k + i uses offset k); waits for all of them before the
// block ends.
template <int OFF0, int OFF1, int OFF2, int OFF3>
MXFA_DEV void lds_read_tr16_4x4(u32x2_t (&r)[16], const uint32_t (&a)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:%20\n\t"
        "ds_read_b64_tr_b16 %1, %17 offset:%20\n\t"
        "ds_read_b64_tr_b16 %2, %18 offset:%20\n\t"
        "ds_read_b64_tr_b16 %3, %19 offset:%20\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:%21\n\t"
        "ds_read_b64_tr_b16 %5, %17 offset:%21\n\t"
        "ds_read_b64_tr_b16 %6, %18 offset:%21\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:%21\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%22\n\t"
        "ds_read_b64_tr_b16 %9, %17 offset:%22\n\t"
        "ds_read_b64_tr_b16 %10, %18 offset:%22\n\t"
        "ds_read_b64_tr_b16 %11, %19 offset:%22\n\t"
        "ds_read_b64_tr_b16 %12, %16 offset:%23\n\t"
        "ds_read_b64_tr_b16 %13, %17 offset:%23\n\t"
        "ds_read_b64_tr_b16 %14, %18 offset:%23\n\t"
        "ds_read_b64_tr_b16 %15, %19 offset:%23\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
          "=&v"(r[15])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF0), "i"(OFF1), "i"(OFF2), "i"(OFF3)
        : "memory");
}

// 16-byte LDS read through a pointer into a __shared__ object (keeps the
// object's identity, so the read waits only for LDS-bound loads into it).
// Sixteen transposing reads: addresses a[0..7] at offset OFF0, then a[0..7]
// at offset OFF1; waits for all of them before the block ends.
template <int OFF0, int OFF1>
MXFA_DEV void lds_read_tr16_x16(u32x2_t (&r)[16], const uint32_t (&a)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %2, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %3, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %5, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %6, %22 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %23 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%25\n\t"
        "ds_read_b64_tr_b16 %9, %17 offset:%25\n\t"
        "ds_read_b64_tr_b16 %10, %18 offset:%25\n\t"
        "ds_read_b64_tr_b16 %11, %19 offset:%25\n\t"
        "ds_read_b64_tr_b16 %12, %20 offset:%25\n\t"
        "ds_read_b64_tr_b16 %13, %21 offset:%25\n\t"
        "ds_read_b64_tr_b16 %14, %22 offset:%25\n\t"
        "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
          "=&v"(r[15])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF0), "i"(OFF1)
        : "memory");
}

MXFA_DEV u32x4_t lds_read16(const void* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(to_lds(const_cast<void*>(p)));
}

MXFA_DEV u32x4_t lds_load16(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((size_t)addr);
}

// Combine a value with the one of lane l ^ 32 (the two halves of the wave
// swapped in registers with v_permlane32_swap; no LDS instruction, so the
// compiler's count of outstanding LDS reads stays exact across branches).
MXFA_DEV float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
MXFA_DEV float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

MXFA_DEV bool wave_any(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }


// ---------------------------------------------------------------- work mapping

// Workgroup -> (batch, query head, q tile), longest work first, XCD aware.
// Workgroups are handed to the 8 XCDs round-robin by linear id, so id i runs
// on XCD i % 8. KV groups (batch, kv head) are dealt to the XCDs round-robin
// (group g -> XCD g % 8), so every XCD gets a share of every sequence, and the
// query heads of one kv group stay on one XCD, where they share K/V in its
// L2. Each XCD walks its items by q tile from the last (most keys under a
// causal mask) to the first.
//
// Within an XCD the hardware places work groups on its CUs round-robin, so
// with two groups per CU the n-th and (n + C)-th groups of an XCD (C = CUs per
// XCD) share a CU for the whole first round. pair_span = C (0: off) mirrors
// the second half of that round: position n in [C, 2C) takes item 3C - 1 - n,
// so each CU starts with a long and a short item of the first 2C instead of
// two similar ones; later positions keep the longest-first order.
struct WorkItem {
    int b;      // batch / segment, or -1 for a padding workgroup
    int h;      // query head
    int qtile;
};

MXFA_DEV WorkItem map_workgroup(int id, int batch, int heads_kv, int group, int n_qtiles, int pair_span = 0) {
    const int x = id % kXcds;
    int n = id / kXcds;
    const int groups = batch * heads_kv;
    const int groups_per_xcd = (groups + kXcds - 1) / kXcds;
    const int per_rank = groups_per_xcd * group;
    if (pair_span > 0 && per_rank * n_qtiles >= 2 * pair_span && n >= pair_span && n < 2 * pair_span)
        n = 3 * pair_span - 1 - n;
    const int rank = n / per_rank;
    const int rem = n % per_rank;
    const int g = (rem / group) * kXcds + x;
    WorkItem w;
    w.qtile = n_qtiles - 1 - rank;
    if (g >= groups || rank >= n_qtiles) {
        w.b = -1;
        w.h = 0;
        return w;
    }
    w.b = g / heads_kv;
    w.h = (g % heads_kv) * group + rem % group;
    return w;
}

// Grid size for map_workgroup.
inline long long workgroup_count(int batch, int heads_kv, int group, int n_qtiles) {
    const long long groups = (long long)batch * heads_kv;
    return (long long)kXcds * ((groups + kXcds - 1) / kXcds) * group * n_qtiles;
}

// Workgroup -> (segment, query head, q tile) of a packed problem from its
// work list (count, prefix sums, then (segment, q tile) pairs ordered by the
// key tiles they stream, most first). Units (list entry e, kv head g), in
// list order, are dealt to the XCDs round-robin; each unit's query heads run
// as consecutive work groups of one XCD, where they share that K/V in its L2.
// pair_span as for map_workgroup. Work groups past the list's end get b = -1.
MXFA_DEV WorkItem map_listed(int id, const int* ws, int batch, int heads_kv, int group, long long list_max,
                             int pair_span = 0) {
    const int x = id % kXcds;
    int n = id / kXcds;
    const long long per_xcd = (list_max * heads_kv + kXcds - 1) / kXcds * group;
    if (pair_span > 0 && per_xcd >= 2 * pair_span && n >= pair_span && n < 2 * pair_span)
        n = 3 * pair_span - 1 - n;
    const long long u = (long long)(n / group) * kXcds + x;
    const long long e = u / heads_kv;
    WorkItem w;
    w.b = -1;
    w.h = 0;
    w.qtile = 0;
    const int count = ws[0];
    if (e >= count) return w;
    const int2 it = reinterpret_cast<const int2*>(ws + 4 + ((batch + 2) & ~1))[e];
    w.b = it.x;
    w.qtile = it.y;
    w.h = (int)(u % heads_kv) * group + n % group;
    return w;
}

// Grid size for map_listed.
inline long long listed_workgroup_count(int heads_kv, int group, long long list_max) {
    return (long long)kXcds * ((list_max * heads_kv + kXcds - 1) / kXcds) * group;
}

}  // namespace mxfa
