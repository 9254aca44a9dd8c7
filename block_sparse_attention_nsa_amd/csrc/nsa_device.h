// nsa_device.h -- device-side building blocks shared by the gfx950 kernels of
// libnsa_sel: problem geometry, bf16 conversions, the 16x16x32 bf16 matrix-core
// (MFMA) step, wavefront shuffles and wave-local LDS ordering.
//
// MFMA lane layouts used throughout (v_mfma_f32_16x16x32_bf16, one wave):
//   A (16 x 32):  lane l holds A[l % 16][8 * (l / 16) + e],  e = 0..7
//   B (32 x 16):  lane l holds B[8 * (l / 16) + e][l % 16],  e = 0..7
//   C (16 x 16):  lane l holds C[4 * (l / 16) + i][l % 16],  i = 0..3
// The contraction index k only has to be laid out the same way in A and B, so
// every kernel is free to pick which 8 k-values lane group g = l / 16 carries.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element strides of one tensor: batch entry (dense only), head, token.  The
// last dimension (D) is contiguous.  Packed tensors have their sequences back
// to back along the token dimension.  The host checks that one batch entry
// spans less than 2^31 elements, so offsets inside an entry are 32-bit.
struct TLayout {
    int64_t sb;
    int32_t sh, st;
};

// Everything a kernel needs to know about the problem (passed by value).
struct Problem {
    int B, T, Hq, Hkv, G, D, S, bs;
    int Tk;       // dense: keys per (batch entry, KV head), >= T (queries are the last T positions)
    int Z;        // batch entries (dense) or sequences (packed)
    int packed;   // 1 when cu is a cumulative-length array
    int Tmax;     // longest sequence of queries (T for dense)
    int NBmax;    // key blocks of the longest sequence (dense: ceil(Tk / bs))
    int Smin;     // min(S, NBmax): distinct usable entries per row, at most
    float scale;  // softmax scale
    float scale_log2;  // scale * log2(e): scores in the base-2 domain
    const int* cu;
    const float* sink;  // [Hq] per-head sink logits (natural log), or null
    int window;         // sliding window: keys t - window < j <= t; 0 = none
    int strided;        // the layouts below were declared by the caller
    // Layouts of q, k, v, o, dO, dq, dk, dv (lse / delta are contiguous).
    TLayout lq, lk, lv, lo, ldo, ldq, ldk, ldv;
};

// Where sequence z lives: its first token along the token dimension (packed)
// and its batch entry (dense).  Packed lengths are clamped so every access
// stays inside the T-token arrays whatever cu holds.  block_idx rows and
// lse / delta entries are counted in their own (contiguous) arrays.
struct Seq {
    int start, len;    // first token (packed) and number of queries
    int klen;          // keys (dense: Tk; packed: len)
    int qoff;          // key position of query 0: query t is at t + qoff (klen - len)
    int zb;            // batch entry of the dense layouts (0 when packed)
    int64_t i_base;    // block_idx row of (hkv, t) = i_base + hkv*T + t
    int64_t l_base;    // lse/delta index of (h, t)  = l_base + h*T + t
};

__device__ __forceinline__ Seq seq_of(const Problem& p, int z) {
    Seq s;
    if (p.packed) {
        int a = p.cu[z], b = p.cu[z + 1];
        a = min(max(a, 0), p.T);
        b = min(max(b, a), p.T);
        s.start = a;
        s.len = min(b - a, p.Tmax);
        s.klen = s.len;
        s.qoff = 0;
        s.zb = 0;
        s.i_base = a;
        s.l_base = a;
    } else {
        s.start = 0;
        s.len = p.T;
        s.klen = p.Tk;
        s.qoff = p.Tk - p.T;
        s.zb = z;
        s.i_base = (int64_t)z * p.Hkv * p.T;
        s.l_base = (int64_t)z * p.Hq * p.T;
    }
    return s;
}

// Element offset of row (h, t) of sequence s in a tensor of layout L, and of
// its token-0 row (the base the token stride is added to).
__device__ __forceinline__ int64_t row_off(const TLayout& L, const Seq& s, int h, int t) {
    return (int64_t)s.zb * L.sb + (h * L.sh + (s.start + t) * L.st);
}
__device__ __forceinline__ int64_t head_base(const TLayout& L, const Seq& s, int h) {
    return row_off(L, s, h, 0);
}
__device__ __forceinline__ int64_t l_off(const Problem& p, const Seq& s, int h, int t) {
    return s.l_base + (int64_t)h * p.T + t;
}
__device__ __forceinline__ const int* idx_row(const Problem& p, const Seq& s, const int* idx,
                                              int hkv, int t) {
    return idx + (s.i_base + (int64_t)hkv * p.T + t) * p.S;
}
// First entry of the (z, hkv) region of the inverted token lists.
__device__ __forceinline__ int64_t region_base(const Problem& p, const Seq& s, int hkv) {
    return (s.i_base + (int64_t)hkv * p.T) * p.Smin;
}

// ---- bf16 ---------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// float -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 converts
// two values per instruction (NaN stays NaN).
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS transposing read (ds_read_b64_tr_b16).  Inside each 16-lane group,
// lane 4r + c passes the address of 4 consecutive bf16 of "row" r
// (Tile[row_r][n0 + 4c .. 4c + 3]); lane i of the group then receives the
// column {Tile[row_r][n0 + i] : r = 0..3}.  Two such reads give one MFMA
// operand whose contraction index runs over 8 rows of a row-major tile.
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* lds_ptr) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr));
    return __builtin_bit_cast(uint2, r);
}

// Operand A[m][k] = Tile[rows(k)][col0 + m] (or B[k][n] = Tile[rows(k)][col0 + n])
// for the 8 rows rows(8g + e) = row_lo + 4g + e (e < 4), row_hi + 4g + e - 4
// (e >= 4) of a row-major bf16 tile with `stride` elements per row.
__device__ __forceinline__ bf16x8 lds_col_operand(const uint16_t* tile, int stride, int row_lo,
                                                  int row_hi, int col0, int lane) {
    int g = lane >> 4, j = lane & 15, r = j >> 2, c = j & 3;
    uint2 lo = lds_read_tr(tile + (row_lo + 4 * g + r) * stride + col0 + 4 * c);
    uint2 hi = lds_read_tr(tile + (row_hi + 4 * g + r) * stride + col0 + 4 * c);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Raw buffer access: a wave-uniform descriptor (base, size in bytes) and a
// 32-bit per-lane byte offset.  Loads whose lane offset (+ immediate) lies
// at or past the size return zeros, so a descriptor that ends at the last
// valid row reads rows past it as 0.  (The scalar offset is not range
// checked; it is only used for in-range strides.)
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

// The base and size must be wave-uniform; readfirstlane states it so the
// compiler keeps the descriptor in SGPRs (no per-lane waterfall loop).
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* b = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(b, (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(buf_rsrc r, int voff, int soff) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

// ---- 32-row tiles staged in LDS by buffer-to-LDS loads ---------------------
// A 32-row x D bf16 tile, rows unpadded (each 1 KB buffer-to-LDS load fills
// 1 KB of consecutive LDS: lane l writes bytes 16 l .. 16 l + 15), with the
// 16-byte chunks of every row permuted so that both operand reads -- 16 rows
// x one chunk (ds_read_b128) and 4 rows x 16 columns (ds_read_b64_tr_b16) --
// spread evenly over the LDS banks.  The permutations were chosen by
// measuring those two access patterns on gfx950 (a rotation by two chunks per
// row for 256-byte rows, XOR swizzles for the shorter ones).
template <int D>
struct RowTile {
    static constexpr int QCH = D / 8;       // 16-byte chunks per row
    static constexpr int RB = 2 * D;        // bytes per row
    static constexpr int TB = 32 * RB;      // bytes per tile
    static constexpr int NI = TB / 1024;    // 1 KB loads per tile
    // LDS slot of data chunk c of row r, and its inverse.
    __host__ __device__ static constexpr int slot(int r, int c) {
        return D == 128 ? ((c + 2 * r) & 15) : D == 64 ? (c ^ (r & 7)) : (c ^ ((r >> 1) & 3));
    }
    __host__ __device__ static constexpr int chunk(int r, int s) {
        return D == 128 ? ((s - 2 * r) & 15) : D == 64 ? (s ^ (r & 7)) : (s ^ ((r >> 1) & 3));
    }
    // Byte offset of this lane's A operand (rows r = lane & 15, columns
    // 32 kk + 8 (lane >> 4) .. + 7): one ds_read_b128; rows 16.. sit 16 RB
    // further with the same slots.
    __device__ static uint32_t a_off(int lane, int kk) {
        const int r = lane & 15, g = lane >> 4;
        return (uint32_t)(r * RB + 16 * slot(r, 4 * kk + g));
    }
    // Byte offset of this lane's transposed read (ds_read_b64_tr_b16) of rows
    // 4 (lane >> 4) + (lane & 15) / 4, columns 16 dt + 4 (lane & 3) .. + 3.
    __device__ static uint32_t t_off(int lane, int dt) {
        const int rr = 4 * (lane >> 4) + ((lane & 15) >> 2), c = lane & 3;
        return (uint32_t)(rr * RB + 16 * slot(rr, 2 * dt + (c >> 1)) + 8 * (c & 1));
    }
    static_assert(slot(16, 0) == slot(0, 0) && slot(17, 3) == slot(1, 3) && slot(31, 5) == slot(15, 5),
                  "rows 16.. repeat the slots of rows 0..");
};

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from the buffer into LDS at dst + 16 * lane.
__device__ __forceinline__ void dma16(buf_rsrc r, void* dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)voff, 0, 0, 0);
}
// 4 bytes per lane into LDS at dst + 4 * lane.
__device__ __forceinline__ void dma4(buf_rsrc r, void* dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, (int)voff, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (they complete in issue order) and its LDS writes are done, then a
// workgroup barrier.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.  Buffers written by buffer-to-LDS loads
// are separate __shared__ variables, so the compiler can tell an access to
// one stage from an in-flight load into another and adds no wait of its own.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const int* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int*)p;
}

// Waits of spin_ge that gave up, per source file that waits (each file has
// its own copy; nsa_sel_wait_timeouts() reads them).  Never expected: a
// nonzero count means a launch computed from a stage that may not have been
// complete.
static __device__ unsigned int g_wait_timeouts;

// Waits until the LDS counter reaches target.  Callers make sure the waves
// that add to it always get there, so the wait ends; the iteration cap only
// bounds it should that ever fail, and then the wave sets the workgroup's
// LDS flag *fail (a plain LDS store on that path only: nothing is carried
// through the callers' loops).  After its loop each wave passes the flag to
// report_wait_timeouts, which counts it in g_wait_timeouts.  The counter is
// read with a plain ds_read_b32 in asm: to the compiler it is unrelated to
// the stages that buffer-to-LDS loads are filling, so it adds no
// vector-memory wait.
__device__ __forceinline__ void spin_ge(const int* ctr, int target, int* fail) {
    const uint32_t a = lds_addr(ctr);
    // (Not unrolled: eight copies per call site bloated the ring loops.)
#pragma nounroll
    for (int it = 0; it < (1 << 18); ++it) {
        int v;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
        if (__builtin_amdgcn_readfirstlane(v) >= target) return;
    }
    asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(fail)), "v"(1) : "memory");
}
// Counts a wave's view of its workgroup's give-up flag (after its loop).
__device__ __forceinline__ void report_wait_timeouts(const int* fail) {
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(fail)) : "memory");
    if (__builtin_amdgcn_readfirstlane(v) != 0 && __lane_id() == 0) atomicAdd(&g_wait_timeouts, 1u);
}

// One count from this wave (LDS operations of a wave are processed in order,
// so its earlier LDS reads and writes are done first).
__device__ __forceinline__ void signal(int* ctr, int lane) {
    if (lane == 0) asm volatile("ds_add_u32 %0, %1" : : "v"(lds_addr(ctr)), "v"(1) : "memory");
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// ---- wavefront helpers ----------------------------------------------------

__device__ __forceinline__ float shfl_xor(float v, int mask) {
    int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

// Wave-uniform tests of a per-lane condition, decided on the scalar unit
// (ballot against exec: no vector compare / select / readfirstlane chain).
__device__ __forceinline__ bool wave_all(bool c) {
    return __builtin_amdgcn_ballot_w64(c) == __builtin_amdgcn_read_exec();
}
__device__ __forceinline__ bool wave_any(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0ull; }
// A value the caller knows to be wave-uniform, moved to scalar registers.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Float max as the bare instruction.  fmaxf obliges the compiler to quiet a
// signalling NaN first, i.e. an extra v_max_f32 x, x on every operand it
// cannot prove canonical (all permlane results, every loop-carried value);
// the scores these kernels take the max of are never NaN.
__device__ __forceinline__ float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (one C-layout column),
// with gfx950's lane-half swaps (v_permlane32_swap exchanges lanes 32..63 of
// one operand with lanes 0..31 of the other, v_permlane16_swap the odd rows
// of 16 lanes with the even ones): each lane ends up holding its own value
// and its partner's, one in each result.
__device__ __forceinline__ float col_max4(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float m = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t um = __float_as_uint(m);
    const auto b = __builtin_amdgcn_permlane16_swap(um, um, false, false);
    return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum4(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t um = __float_as_uint(m);
    const auto b = __builtin_amdgcn_permlane16_swap(um, um, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Order this wave's LDS accesses: everything issued before is complete and
// visible to the wave before anything after it runs.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// A finished softmax row with an attention-sink logit sk (natural log) in
// its denominator: m2 is the row's running max in base-2 units and l the sum
// of 2^(x - m2) over its keys (l = 0: no key).  Gives the factor that
// normalises the output accumulated relative to 2^m2 and the row's lse:
// with M = max(m2, sk log2 e), L = l 2^(m2 - M) + 2^(sk log2 e - M),
// inv = 2^(m2 - M) / L and lse = (M + log2 L) ln 2 (a row with no key gets
// o = 0, lse = sk; a sink of -inf changes nothing).
__device__ __forceinline__ void finish_row_sink(float sk, float m2, float l, float& inv, float& lse) {
    const float ninf = -__builtin_huge_valf();
    const float mk = l > 0.f ? m2 : ninf;
    const float s2 = sk * kLog2e;
    const float M = fmaxf(mk, s2);
    if (M == ninf) {
        inv = 0.f;
        lse = ninf;
        return;
    }
    const float a = mk == ninf ? 0.f : fast_exp2(mk - M);
    const float L = l * a + (s2 == ninf ? 0.f : fast_exp2(s2 - M));
    inv = a / L;
    lse = (M + fast_log2(L)) * kLn2;
}

// Workgroup index remapped so that consecutive logical indices stay on one
// XCD (the dispatcher deals workgroups round-robin over the 8 XCDs, each
// with its own L2): logical ranges then share K/V in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int X = 8;
    int xcd = bid % X, k = bid / X;
    int q = n / X, r = n % X;
    return xcd * q + min(xcd, r) + k;
}

}  // namespace nsa
