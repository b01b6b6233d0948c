// Fused radiance-network evaluation on the gfx950 matrix cores.
//
// One wave evaluates the network on 32*SB samples (bf16: 64, f32: 32).
// Activations never leave registers: a layer's accumulators are rounded
// (bf16) or copied (f32) straight into the B operands of the next layer
// (layout in nets.hpp).  Weight tiles are read from the packed buffer in
// the order the layer loops consume them.  Layers run output-block major so
// only 32*SB accumulators are live at a time, next to the input and output
// activations of the layer.
#pragma once

#include "common.hpp"
#include "nets.hpp"

namespace nerf {

template <int V>
struct IntC {
    static constexpr int value = V;
};

// Calls f(IntC<I>) for I = B..E-1 in order, fully unrolled.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(IntC<B>{});
        static_for<B + 1, E>(f);
    }
}

struct TBF16 {
    static constexpr int prec = PREC_BF16;
    static constexpr int SB = 2;
    using Op = bf16x8;
    __device__ static __forceinline__ f32x16 mma(Op a, Op b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

// bfloat16 with one sample block of 32 per wave: half the registers of
// TBF16, for kernels that need two waves per SIMD.
struct TBF16S1 {
    static constexpr int prec = PREC_BF16;
    static constexpr int SB = 1;
    using Op = bf16x8;
    __device__ static __forceinline__ f32x16 mma(Op a, Op b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

struct TF32 {
    static constexpr int prec = PREC_F32;
    static constexpr int SB = 1;
    using Op = float;
    __device__ static __forceinline__ f32x16 mma(Op a, Op b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

#define NERF_AS_GLOBAL __attribute__((address_space(1)))
#define NERF_AS_LDS __attribute__((address_space(3)))
#define NERF_AS_CONST __attribute__((address_space(4)))

// Compiler-only memory fence: no instruction, but no memory access moves
// across it.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt vmcnt(VM) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
}
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// ---------------------------------------------------------------------------
// Weight streams.  A network's tiles are consumed strictly in packed order,
// tile t at byte t*TB of the tile region, and get<t>() is only ever called
// with compile-time t, in increasing order, once per forward pass.
// ---------------------------------------------------------------------------

// LdsStream: the 4 waves of a 256-thread workgroup share one ring of NBUF
// LDS slots of kChunkBytes each.  Chunk k of the tile region is copied
// global->LDS by direct loads (each wave moves a quarter of it, no VGPRs)
// into slot k % NBUF, NBUF-1 chunks ahead of its use.  At the first tile of
// chunk k every wave waits until its own copies of chunk k have landed and
// its reads of chunk k-1 are done, the workgroup meets at a barrier, and
// chunk k+NBUF-1 is issued into the slot chunk k-1 used.  Every wave of the
// workgroup must run the same sequence of forward passes.
#ifndef NERF_CHUNK_KB
#define NERF_CHUNK_KB 16
#endif
constexpr int kChunkBytes = NERF_CHUNK_KB * 1024;
static_assert(kTileRegionAlign % kChunkBytes == 0, "chunks tile the padded weight region");
constexpr int kChunkDma = kChunkBytes / 1024 / 4;  // 1 KB copies per wave per chunk

static __shared__ __attribute__((aligned(1024))) char g_ring0[kChunkBytes];
static __shared__ __attribute__((aligned(1024))) char g_ring1[kChunkBytes];
static __shared__ __attribute__((aligned(1024))) char g_ring2[kChunkBytes];
static __shared__ __attribute__((aligned(1024))) char g_ring3[kChunkBytes];
static __shared__ __attribute__((aligned(1024))) char g_ring4[kChunkBytes];
static __shared__ __attribute__((aligned(1024))) char g_ring5[kChunkBytes];
static __shared__ __attribute__((aligned(1024))) char g_ring6[kChunkBytes];
static __shared__ __attribute__((aligned(1024))) char g_ring7[kChunkBytes];

template <int S>
__device__ __forceinline__ char* ring_slot() {
    static_assert(S >= 0 && S < 8, "ring slot");
    if constexpr (S == 0) return g_ring0;
    else if constexpr (S == 1) return g_ring1;
    else if constexpr (S == 2) return g_ring2;
    else if constexpr (S == 3) return g_ring3;
    else if constexpr (S == 4) return g_ring4;
    else if constexpr (S == 5) return g_ring5;
    else if constexpr (S == 6) return g_ring6;
    else return g_ring7;
}

#ifndef NERF_LOOK
#define NERF_LOOK 3
#endif
template <class T, int KIND, int NBUF, int LOOK = NERF_LOOK>
struct LdsStream {
    static_assert(NBUF >= 2 && NBUF <= 8, "ring depth");
    using Op = typename T::Op;
    static constexpr int TB = tile_bytes(T::prec);
    static constexpr size_t BYTES = net_tiles_bytes(KIND, T::prec);
    static constexpr int NT = (int)(BYTES / TB);               // tiles
    static constexpr int NCH = (int)((BYTES + kChunkBytes - 1) / kChunkBytes);
    __amdgpu_buffer_rsrc_t rsrc;  // the padded tile region; reads past it return zero
    int voff;                     // this lane's byte offset within a chunk
    int dst;                      // this wave's byte offset within a slot
    int lane;
    Op buf[LOOK];                 // tiles t..t+LOOK-1, read ahead of use

    // Each wave copies kChunkDma consecutive kilobytes of every chunk.
    __device__ __forceinline__ LdsStream(const char* packed, int lane_, int wave)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(packed), (short)0,
                                                 (int)net_tiles_padded(KIND, T::prec), kBufferWord3)),
          voff(wave * (kChunkDma * 1024) + lane_ * 16), dst(wave * (kChunkDma * 1024)), lane(lane_) {}

    // One copy of kilobyte I of this wave's share of chunk K, as a buffer load
    // into LDS: the chunk offset is the scalar offset, the lane's offset a
    // VGPR fixed for the whole stream, the piece the immediate offset (which
    // moves the LDS address too), and all pieces of a chunk share one LDS
    // base (M0).  (A new M0 per piece makes each copy wait for the previous
    // one to leave the wave.  The buffer form, unlike the global one, also
    // lets the compiler keep counting LDS reads in order, so tile reads stay
    // in flight across the copies.)
    template <int K, int I>
    __device__ __forceinline__ void piece() {
        static_assert(I * 1024 < 4096, "immediate offset range");
        if constexpr (K < NCH) {
            char* slot = ring_slot<K % NBUF>() + dst;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (NERF_AS_LDS void*)slot, 16, voff, K * kChunkBytes, I * 1024,
                                                     0);
        }
    }
    template <int K>
    __device__ __forceinline__ void issue() {
        static_for<0, kChunkDma>([&](auto i) { piece<K, i.value>(); });
    }

    template <int K>
    __device__ __forceinline__ void boundary() {
        constexpr int ahead = (NCH - 1 - K) < (NBUF - 2) ? (NCH - 1 - K) : (NBUF - 2);
        wait_vm_lgkm0<ahead * kChunkDma>();
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        issue<K + NBUF - 1>();
    }

    template <int TILE>
    __device__ __forceinline__ Op read() {
        constexpr int off = TILE * TB;
        constexpr int K = off / kChunkBytes;
        if constexpr (off % kChunkBytes == 0) boundary<K>();
        const char* p = ring_slot<K % NBUF>() + (off % kChunkBytes) + lane * (int)sizeof(Op);
        return *reinterpret_cast<const Op*>(p);
    }

    // Start of a forward pass: every wave is done with the previous pass's
    // slots and has no vector memory operation in flight; issue the first
    // NBUF-1 chunks and read the first LOOK tiles.
    __device__ __forceinline__ void begin() {
        wait_all();
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        static_for<0, NBUF - 1>([&](auto k) { issue<k.value>(); });
        static_for<0, LOOK>([&](auto t) {
            if constexpr (t.value < NT) buf[t.value] = read<t.value>();
        });
    }

    template <int TILE>
    __device__ __forceinline__ Op get() {
        const Op cur = buf[TILE % LOOK];
        if constexpr (TILE + LOOK < NT) buf[TILE % LOOK] = read<TILE + LOOK>();
        return cur;
    }
};

// GlobalStream: each wave reads its tiles straight from global memory (for
// waves that evaluate different networks), LOOK tiles ahead of use.
template <class T, int KIND, int LOOK = 6>
struct GlobalStream {
    using Op = typename T::Op;
    static constexpr int TB = tile_bytes(T::prec);
    static constexpr int NT = (int)(net_tiles_bytes(KIND, T::prec) / TB);  // real tiles, no padding
    const NERF_AS_GLOBAL char* base;  // this lane's bytes of tile 0
    Op buf[LOOK];
    __device__ __forceinline__ GlobalStream(const char* packed, int lane, int)
        : base((const NERF_AS_GLOBAL char*)packed + lane * (int)sizeof(Op)) {}
    template <int TILE>
    __device__ __forceinline__ Op read() const {
        return *reinterpret_cast<const NERF_AS_GLOBAL Op*>(base + TILE * TB);
    }
    __device__ __forceinline__ void begin() {
        static_for<0, LOOK>([&](auto t) {
            if constexpr (t.value < NT) buf[t.value] = read<t.value>();
        });
    }
    template <int TILE>
    __device__ __forceinline__ Op get() {
        const Op cur = buf[TILE % LOOK];
        if constexpr (TILE + LOOK < NT) buf[TILE % LOOK] = read<TILE + LOOK>();
        return cur;
    }
};

// Biases.  A network's bias region (all layers, [ob][half][16] float32) is
// copied once per workgroup into LDS; a lane reads the 16 biases of its half
// of an output block with broadcast LDS reads, in order with the tile reads.
template <int KIND, int PREC>
struct BiasRegion {
    static constexpr size_t begin = net_bias_offset(KIND, PREC, 0);
    static constexpr size_t bytes = net_packed_bytes(KIND, PREC) - begin;
    static constexpr int floats = (int)(bytes / sizeof(float));
    template <int LAYER>
    static constexpr int layer_float() {
        return (int)((net_bias_offset(KIND, PREC, LAYER) - begin) / sizeof(float));
    }
    static constexpr int layer_float_rt(int layer) {
        return (int)((net_bias_offset(KIND, PREC, layer) - begin) / sizeof(float));
    }
};

// Copies the bias region of a packed network to LDS; every thread of the
// workgroup takes part; the caller synchronises the workgroup afterwards.
template <int KIND, int PREC>
__device__ __forceinline__ void bias_to_lds(NERF_AS_LDS float* dst, const char* packed, int tid, int nthreads) {
    using BR = BiasRegion<KIND, PREC>;
    const f32x4* src = reinterpret_cast<const f32x4*>(packed + BR::begin);
    for (int i = tid; i < BR::floats / 4; i += nthreads) reinterpret_cast<NERF_AS_LDS f32x4*>(dst)[i] = src[i];
}

// Four 16-byte reads, not one 64-byte read: the compiler splits a 64-byte LDS
// read into four without keeping its alias information, then cannot tell it
// apart from the weight ring's direct loads and waits for every one of them
// in flight (vmcnt(0)) before the read.
__device__ __forceinline__ f32x16 load_bias16(const NERF_AS_LDS float* bias, int layer_float, int ob, int h) {
    const NERF_AS_LDS f32x4* p = reinterpret_cast<const NERF_AS_LDS f32x4*>(bias + layer_float) + 4 * (2 * ob + h);
    const f32x4 q0 = p[0], q1 = p[1], q2 = p[2], q3 = p[3];
    return f32x16{q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3],
                  q2[0], q2[1], q2[2], q2[3], q3[0], q3[1], q3[2], q3[3]};
}

// Global-memory variant, for waves that each evaluate a different network
// (the bias pointer is the start of that network's bias region).
__device__ __forceinline__ f32x16 load_bias16(const float* bias, int layer_float, int ob, int h) {
    return ((const NERF_AS_GLOBAL f32x16*)(bias + layer_float))[2 * ob + h];
}

template <class T, int KIND, int LAYER>
struct LayerInfo {
    static constexpr Layer L = net_layers(KIND)[LAYER];
    static constexpr int S1 = seg_steps(L.s0, T::prec);
    static constexpr int S2 = seg_steps(L.s1, T::prec);
    static constexpr int OB = out_blocks(L.n_out);
    static constexpr int tile0 = (int)(net_tile_offset(KIND, T::prec, LAYER) / tile_bytes(T::prec));
    static constexpr int bias = BiasRegion<KIND, T::prec>::template layer_float<LAYER>();
};

// Steps of the output of LAYER as an input of the next layer.
template <class T, int KIND, int LAYER>
constexpr int out_steps() {
    return seg_steps(Seg{SEG_HIDDEN, net_layers(KIND)[LAYER].n_out, 0}, T::prec);
}


// ReLU on the bit pattern: negative floats are negative integers, so one
// integer max clamps them to +0.
template <bool RELU>
__device__ __forceinline__ float act(float v) {
    if constexpr (RELU) {
        return __builtin_bit_cast(float, max(__builtin_bit_cast(int, v), 0));
    } else {
        return v;
    }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Places a bf16x8 operand in accumulation registers: matrix instructions
// read their A/B operands from them directly, which leaves the
// architectural registers to the weight tiles in flight and the epilogue.
__device__ __forceinline__ bf16x8 to_agpr(bf16x8 v) {
    i32x4 bits = __builtin_bit_cast(i32x4, v);
    asm volatile("" : "+a"(bits));
    return __builtin_bit_cast(bf16x8, bits);
}
__device__ __forceinline__ float to_agpr(float v) {
    asm volatile("" : "+a"(v));
    return v;
}

// Epilogue of one output block, cut into pieces so it can run between the
// matrix instructions of the next block.  bf16: piece p = (sb, q) turns 8
// accumulators into one operand of the next layer; f32: piece p copies
// accumulator p.
template <class T>
struct Epi;
template <int NSB>
struct EpiBf16 {
    // The epilogue in 4 units per sample block for the slots between matrix
    // instructions: piece p = (sb, q) turns 8 accumulators into one operand
    // of the next layer; unit 2p rounds, packs and rectifies piece p into
    // VGPRs (8 VALU), unit 2p+1 moves it to the AGPR operand of the next
    // layer (4 writes).
    static constexpr int units = 4 * NSB;
    struct Tmp {
        i32x4 t;
    };
    template <int U, bool RELU, class Out>
    __device__ static __forceinline__ void unit(const f32x16 (&acc)[NSB], Out& out, int ob, Tmp& tmp) {
        constexpr int P = U / 2, sb = P / 2, q = P % 2;
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        typedef short i16x2 __attribute__((ext_vector_type(2)));
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        if constexpr (U % 2 == 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x2 f = {acc[sb][8 * q + 2 * c], acc[sb][8 * q + 2 * c + 1]};
                i16x2 w = __builtin_bit_cast(i16x2, __builtin_convertvector(f, bf16x2));
                if constexpr (RELU) w = __builtin_elementwise_max(w, i16x2{0, 0});
                tmp.t[c] = __builtin_bit_cast(int, w);
            }
        } else {
            i32x4 t = tmp.t;
            asm volatile("" : "+a"(t));
            out[2 * ob + q][sb] = __builtin_bit_cast(bf16x8, t);
        }
    }
};

template <>
struct Epi<TBF16> : EpiBf16<2> {};
template <>
struct Epi<TBF16S1> : EpiBf16<1> {};

template <>
struct Epi<TF32> {
    static constexpr int pieces = 16;
    template <int P, bool RELU, class Out>
    __device__ static __forceinline__ void piece(const f32x16 (&acc)[1], Out& out, int ob) {
        out[16 * ob + P][0] = act<RELU>(acc[0][P]);
    }
    static constexpr int units = 16;
    struct Tmp {};
    template <int U, bool RELU, class Out>
    __device__ static __forceinline__ void unit(const f32x16 (&acc)[1], Out& out, int ob, Tmp&) {
        piece<U, RELU>(acc, out, ob);
    }
};

// Epilogue sources for mma_block: nothing, or a finished block whose
// accumulators still have to become operands of the next layer (block OBP of
// a layer with activation RELU, written into *out).
struct NoEpi {
    static constexpr bool active = false;
    template <int U, class Tmp>
    __device__ __forceinline__ void unit(Tmp&) {}
    __device__ __forceinline__ void finish() {}
};

template <class T, bool RELU, int OBP, class Out>
struct BlockEpi {
    static constexpr bool active = true;
    static constexpr int ob = OBP;
    f32x16 acc[T::SB];
    Out* out;
    template <int U>
    __device__ __forceinline__ void unit(typename Epi<T>::Tmp& tmp) {
        Epi<T>::template unit<U, RELU>(acc, *out, OBP, tmp);
    }
    __device__ __forceinline__ void finish() {
        typename Epi<T>::Tmp tmp{};
        static_for<0, Epi<T>::units>([&](auto u) { unit<u.value>(tmp); });
    }
};

// Slot of epilogue unit u in a block of S steps: with two sample blocks,
// slot 2*st lies between the two MFMAs of step st and slot 2*st+1 after
// them; units use the between-slots when there are enough steps, else every
// slot; with one sample block, units follow the MFMAs.  Slots >= 2*S run
// after the block.
template <class T, int S>
constexpr int epi_slot(int u) {
    constexpr bool TWO = T::SB == 2;
    constexpr bool DENSE = !TWO || S < Epi<T>::units;
    return TWO ? (DENSE ? u : 2 * u) : 2 * u + 1;
}

// True when block OBP's epilogue, run in the first block (S steps) of the
// layer that reads it as its first input segment, writes every operand
// before the MFMA that reads it (program order decides which value an
// operand read sees).  bf16: unit 2p+1 writes operand (step 2*OBP + p%2,
// sample block p/2), read just before slot 2*step + sb (one sample block:
// before slot 2*step, the slot after the previous step's MFMA being
// 2*step - 1).  f32: unit u writes step 16*OBP + u, read before slot
// 2*step + 1.
template <class T, int S, int OBP>
constexpr bool epi_defer_ok() {
    for (int u = 0; u < Epi<T>::units; ++u) {
        const int slot = epi_slot<T, S>(u);
        if (slot >= 2 * S) return false;
        if constexpr (T::prec == PREC_BF16) {
            if (u % 2 == 0) continue;
            const int p = u / 2, k = 2 * OBP + p % 2, sb = p / 2;
            if (k < S && !(slot < 2 * k + sb)) return false;
        } else {
            const int k = 16 * OBP + u;
            if (k < S && !(slot < 2 * k + 1)) return false;
        }
    }
    return true;
}

// acc = W(ob) [in1, in2] + bias; the bias enters as the C operand of the
// first step.  The epilogue units of `epi` run in the slots above, where the
// wave would otherwise wait for the matrix pipe.  Scheduling barriers keep
// each step's tile read, matrix instructions and epilogue units in place, so
// the read-ahead distance and the interleave survive scheduling.
template <class T, int TILE0, int S1, int S2, class In1, class In2, class WS, class E>
__device__ __forceinline__ void mma_block(f32x16 (&acc)[T::SB], const f32x16& bias, const In1& in1, const In2& in2,
                                          WS& ws, E& epi) {
    constexpr int S = S1 + S2;
    constexpr int U = E::active ? Epi<T>::units : 0;
    constexpr bool TWO = T::SB == 2;
    typename Epi<T>::Tmp tmp{};
    auto run_slot = [&](auto slot) {
        static_for<0, U>([&](auto uc) {
            if constexpr (epi_slot<T, S>(uc.value) == decltype(slot)::value) epi.template unit<uc.value>(tmp);
        });
    };
    static_for<0, S>([&](auto sc) {
        constexpr int st = sc.value;
        const typename T::Op a = ws.template get<TILE0 + st>();
        static_for<0, T::SB>([&](auto sbc) {
            constexpr int sb = sbc.value;
            const typename T::Op b = st < S1 ? in1[st < S1 ? st : 0][sb] : in2[st >= S1 ? st - S1 : 0][sb];
            acc[sb] = T::mma(a, b, st == 0 ? bias : acc[sb]);
            __builtin_amdgcn_sched_barrier(0);
            run_slot(IntC<2 * st + (TWO ? sb : 1)>{});
            __builtin_amdgcn_sched_barrier(0);
        });
    });
    static_for<0, U>([&](auto uc) {
        if constexpr (epi_slot<T, S>(uc.value) >= 2 * S) epi.template unit<uc.value>(tmp);
    });
}

// Runs `pin` (the previous layer's last block) inside this layer's first
// block when that is safe (epi_defer_ok), else before it.
template <class T, int S, class P>
__device__ __forceinline__ auto& defer_or_finish(P& pin, NoEpi& none) {
    if constexpr (P::active) {
        if constexpr (epi_defer_ok<T, S, P::ob>()) {
            return pin;
        } else {
            pin.finish();
            return none;
        }
    } else {
        return none;
    }
}

// A hidden layer: out = act(W [in1, in2] + b), kept as next-layer operands.
// b0 holds this layer's first bias (read ahead by the caller) and, on
// return, the first bias of layer NEXT (NEXT < 0: none); pin is the previous
// layer's last block, run inside this layer's first block; the return value
// is this layer's last block, for the next layer to run.
template <class T, int KIND, int LAYER, int NEXT, class In1, class In2, class Out, class WS, class BP, class P>
__device__ __forceinline__ auto dense_layer(const In1& in1, const In2& in2, Out& out, WS& ws, BP bias, int lane,
                                            f32x16& b0, P& pin) {
    using I = LayerInfo<T, KIND, LAYER>;
    constexpr bool RELU = I::L.relu != 0;
    constexpr int S = I::S1 + I::S2;
    const int h = lane >> 5;
    f32x16 prev[T::SB];
    NoEpi none;
    auto& first = defer_or_finish<T, S>(pin, none);
    // each block's bias is read one block ahead, so the first MFMA of a block
    // (bias as its C operand) never waits for it
    f32x16 bnext = b0;
    static_for<0, I::OB>([&](auto obc) {
        constexpr int ob = obc.value;
        const f32x16 b = bnext;
        if constexpr (ob + 1 < I::OB) {
            bnext = load_bias16(bias, I::bias, ob + 1, h);
            compiler_fence();  // issue the reads here, not next to their use
        } else if constexpr (NEXT >= 0) {
            b0 = load_bias16(bias, LayerInfo<T, KIND, NEXT>::bias, 0, h);
            compiler_fence();
        }
        f32x16 acc[T::SB];
        if constexpr (ob == 0) {
            mma_block<T, I::tile0, I::S1, I::S2>(acc, b, in1, in2, ws, first);
        } else {
            BlockEpi<T, RELU, ob - 1, Out> pe{{}, &out};
#pragma unroll
            for (int sb = 0; sb < T::SB; ++sb) pe.acc[sb] = prev[sb];
            mma_block<T, I::tile0 + ob * S, I::S1, I::S2>(acc, b, in1, in2, ws, pe);
        }
#pragma unroll
        for (int sb = 0; sb < T::SB; ++sb) prev[sb] = acc[sb];
    });
    BlockEpi<T, RELU, I::OB - 1, Out> last{{}, &out};
#pragma unroll
    for (int sb = 0; sb < T::SB; ++sb) last.acc[sb] = prev[sb];
    return last;
}

// A head (one output block, no activation): raw accumulators.  b0 and pin as
// for dense_layer.
template <class T, int KIND, int LAYER, int NEXT, class In1, class In2, class WS, class BP, class P>
__device__ __forceinline__ void dense_head(const In1& in1, const In2& in2, f32x16 (&acc)[T::SB], WS& ws, BP bias,
                                           int lane, f32x16& b0, P& pin) {
    using I = LayerInfo<T, KIND, LAYER>;
    static_assert(I::OB == 1, "head layers have one output block");
    NoEpi none;
    auto& first = defer_or_finish<T, I::S1 + I::S2>(pin, none);
    const f32x16 b = b0;
    if constexpr (NEXT >= 0) {
        b0 = load_bias16(bias, LayerInfo<T, KIND, NEXT>::bias, 0, lane >> 5);
        compiler_fence();
    }
    mma_block<T, I::tile0, I::S1, I::S2>(acc, b, in1, in2, ws, first);
}

// ---------------------------------------------------------------------------
// NeRF family: hidden layers 0..D-1 (skip segment where the layer has one),
// then density head D, feature D+1, direction layer D+2, rgb head D+3.
// ---------------------------------------------------------------------------
template <int KIND>
struct NerfFamily {
    static constexpr int D = net_n_layers(KIND) - 4;
    static constexpr int LPOS = net_layers(KIND)[0].s0.L;
    static constexpr int LDIR = net_layers(KIND)[D + 2].s1.L;
};

// Hidden layers I..D-1, alternating between cur and nxt; returns the last
// one's final block (pending epilogue).
template <class T, int KIND, int I, int D, class H, class E, class WS, class BP, class P>
__device__ __forceinline__ auto hidden_chain(H& cur, H& nxt, const E& enc, WS& ws, BP bias, int lane, f32x16& b0,
                                             P& pin) {
    // enc is read only by a skip layer (S2 > 0)
    auto pe = dense_layer<T, KIND, I, I + 1>(cur, enc, nxt, ws, bias, lane, b0, pin);
    if constexpr (I + 1 < D)
        return hidden_chain<T, KIND, I + 1, D>(nxt, cur, enc, ws, bias, lane, b0, pe);
    else
        return pe;
}

// enc: position-encoding operands; denc: direction-encoding operands.
// sig[sb] accumulator 0 and rgb[sb] accumulators 0..2 of lanes 0..31 hold the
// outputs of sample (sb*32 + lane).
template <class T, int KIND, class E, class DE, class WS, class BP>
__device__ __forceinline__ void nerf_forward(const E& enc, const DE& denc, WS& ws, BP bias, f32x16 (&sig)[T::SB],
                                             f32x16 (&rgb)[T::SB], int lane) {
    using Fam = NerfFamily<KIND>;
    constexpr int D = Fam::D;
    static_assert(D >= 2, "at least two hidden layers");
    constexpr int HS = out_steps<T, KIND, 0>();
    constexpr int GS = out_steps<T, KIND, D + 2>();
    typename T::Op hA[HS][T::SB], hB[HS][T::SB];
    ws.begin();
    f32x16 b0 = load_bias16(bias, LayerInfo<T, KIND, 0>::bias, 0, lane >> 5);
    NoEpi none;
    auto p0 = dense_layer<T, KIND, 0, 1>(enc, enc, hA, ws, bias, lane, b0, none);
    auto pl = hidden_chain<T, KIND, 1, D>(hA, hB, enc, ws, bias, lane, b0, p0);
    // the last hidden layer (index D-1) wrote hB when D-1 is odd, else hA
    auto& hl = ((D - 1) % 2 == 1) ? hB : hA;
    auto& hf = ((D - 1) % 2 == 1) ? hA : hB;
    dense_head<T, KIND, D, D + 1>(hl, hl, sig, ws, bias, lane, b0, pl);
    NoEpi none2;
    auto pf = dense_layer<T, KIND, D + 1, D + 2>(hl, hl, hf, ws, bias, lane, b0, none2);
    typename T::Op g[GS][T::SB];
    auto pg = dense_layer<T, KIND, D + 2, D + 3>(hf, denc, g, ws, bias, lane, b0, pf);
    dense_head<T, KIND, D + 3, -1>(g, g, rgb, ws, bias, lane, b0, pg);
}

// ---------------------------------------------------------------------------
// Float32 NeRF family with a runtime loop over layers.  Fully unrolling a
// float32 chain (32x32x2 steps: ~9,300 matrix instructions for 8x256) makes
// compile time explode, so one copy of a layer body serves every layer: up
// to 8 output blocks, each up to 8 hidden k-groups and 2 encoding k-groups
// of 16 steps, skipped at run time where a layer has fewer.  The hidden
// state is read from `hin` and written to `hout`; a layer that is read again
// by the next one copies hout to hin (density head: no copy, the feature
// layer reads the same state).  Weight tiles stream per wave straight from
// global memory (L2) one 16-tile group ahead of use.
// ---------------------------------------------------------------------------
struct LoopLayer {
    int n_ob;        // output blocks
    int n_hkb;       // hidden input k-groups (16 steps each)
    int seg2;        // 0 none, 1 position encoding, 2 direction encoding
    int relu;
    int commit;      // copy hout to hin afterwards
    int save;        // 0 none, 1 density head, 2 rgb head
    int bias_float;  // first bias of the layer in the bias region
};

template <int KIND>
struct LoopPlan {
    using Fam = NerfFamily<KIND>;
    static constexpr int NL = net_n_layers(KIND);
    static constexpr LoopLayer layer(int i) {
        const Layer L = net_layers(KIND)[i];
        LoopLayer d{};
        d.n_ob = out_blocks(L.n_out);
        d.n_hkb = L.s0.kind == SEG_HIDDEN ? seg_steps(L.s0, PREC_F32) / 16 : 0;
        const Seg e = L.s0.kind == SEG_ENC ? L.s0 : L.s1;
        d.seg2 = e.kind != SEG_ENC ? 0 : (e.L == Fam::LPOS && i != Fam::D + 2 ? 1 : 2);
        d.relu = L.relu;
        d.commit = i != Fam::D;
        d.save = i == Fam::D ? 1 : (i == Fam::D + 3 ? 2 : 0);
        d.bias_float = BiasRegion<KIND, PREC_F32>::layer_float_rt(i);
        return d;
    }
    struct Table {
        LoopLayer l[NL];
    };
    static constexpr Table table() {
        Table t{};
        for (int i = 0; i < NL; ++i) t.l[i] = layer(i);
        return t;
    }
    static constexpr bool fits() {
        for (int i = 0; i < NL; ++i) {
            const Layer L = net_layers(KIND)[i];
            if (out_blocks(L.n_out) > 8 || (L.s0.kind == SEG_HIDDEN && seg_steps(L.s0, PREC_F32) > 128)) return false;
            if (L.s0.kind == SEG_HIDDEN && seg_steps(L.s0, PREC_F32) % 16) return false;
        }
        return true;
    }
};

// Weight tiles of the looped float32 network: group g = tiles 16g..16g+15
// (one float per lane each).  cur holds the group in use, nxt the one
// after it; next() moves on and fetches the group after that.
struct F32Groups {
    const NERF_AS_GLOBAL char* base;  // this lane's bytes of tile 0
    int next_tile;                    // first tile of the group in nxt
    int last_group_tile;              // last valid group start (reads never pass the tiles)
    float cur[16], nxt[16];
    __device__ __forceinline__ F32Groups(const char* packed, int lane, int n_tiles)
        : base((const NERF_AS_GLOBAL char*)packed + lane * 4), next_tile(16), last_group_tile(n_tiles - 16) {}
    __device__ __forceinline__ void load(float (&dst)[16], int t) const {
        t = t < last_group_tile ? t : last_group_tile;
        const NERF_AS_GLOBAL char* p = base + (size_t)t * 256;
#pragma unroll
        for (int j = 0; j < 16; ++j) dst[j] = *reinterpret_cast<const NERF_AS_GLOBAL float*>(p + 256 * j);
    }
    __device__ __forceinline__ void begin() {
        load(cur, 0);
        load(nxt, 16);
    }
    __device__ __forceinline__ void next() {
#pragma unroll
        for (int j = 0; j < 16; ++j) cur[j] = nxt[j];
        next_tile += 16;
        load(nxt, next_tile);
    }
};

template <int KIND>
__constant__ typename LoopPlan<KIND>::Table kLoopTable = LoopPlan<KIND>::table();

// Networks whose float32 form runs through the layer loop.
template <class T, int KIND>
constexpr bool kLoopedF32 = T::prec == PREC_F32 && KIND == NET_8x256;

template <int KIND, int ES, int DS>
__device__ __forceinline__ void nerf_forward_f32_loop(const float (&enc)[ES][1], const float (&denc)[DS][1],
                                                      const char* packed, const NERF_AS_LDS float* bias,
                                                      f32x16 (&sig)[1], f32x16 (&rgb)[1], int lane) {
    using P = LoopPlan<KIND>;
    static_assert(P::fits(), "layer shapes of the looped float32 network");
    static_assert(ES % 16 == 0 && ES <= 32 && DS % 16 == 0 && DS <= 32, "encoding segments in whole groups");
    constexpr int NT = (int)(net_tiles_bytes(KIND, PREC_F32) / 256);
    const int h = lane >> 5;
    // matrix-instruction B operands (the layer input and both encodings) sit
    // in accumulation registers; the outputs of a layer are written by
    // vector instructions into architectural registers
    float hin[128], hout[128], pe[ES], de[DS];
#pragma unroll
    for (int i = 0; i < 128; ++i) hin[i] = 0.0f;
#pragma unroll
    for (int i = 0; i < ES; ++i) pe[i] = to_agpr(enc[i][0]);
#pragma unroll
    for (int i = 0; i < DS; ++i) de[i] = to_agpr(denc[i][0]);
    F32Groups ws(packed, lane, NT);
    ws.begin();
    sig[0] = f32x16{};
    rgb[0] = f32x16{};
#pragma unroll 1
    for (int li = 0; li < P::NL; ++li) {
        const LoopLayer L = kLoopTable<KIND>.l[li];
        static_for<0, 8>([&](auto obc) {
            constexpr int ob = obc.value;
            if (ob < L.n_ob) {
                f32x16 acc = load_bias16(bias, L.bias_float, ob, h);
                static_for<0, 8>([&](auto kbc) {
                    constexpr int kb = kbc.value;
                    if (kb < L.n_hkb) {
                        static_for<0, 16>([&](auto j) {
                            acc = TF32::mma(ws.cur[j.value], hin[16 * kb + j.value], acc);
                        });
                        ws.next();
                    }
                });
                if (L.seg2 == 1) {
                    static_for<0, ES / 16>([&](auto g) {
                        static_for<0, 16>([&](auto j) {
                            acc = TF32::mma(ws.cur[j.value], pe[16 * g.value + j.value], acc);
                        });
                        ws.next();
                    });
                } else if (L.seg2 == 2) {
                    static_for<0, DS / 16>([&](auto g) {
                        static_for<0, 16>([&](auto j) {
                            acc = TF32::mma(ws.cur[j.value], de[16 * g.value + j.value], acc);
                        });
                        ws.next();
                    });
                }
                if (ob == 0) {
                    // element-wise selects: a conditional store of the whole
                    // vector would be lowered through private memory
                    const bool s1 = L.save == 1, s2 = L.save == 2;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        sig[0][r] = s1 ? acc[r] : sig[0][r];
                        rgb[0][r] = s2 ? acc[r] : rgb[0][r];
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) hout[16 * ob + r] = L.relu ? fmaxf(acc[r], 0.0f) : acc[r];
            }
        });
        if (L.commit) {
#pragma unroll
            for (int i = 0; i < 128; ++i) hin[i] = to_agpr(hout[i]);
        }
    }
}

// Hash-grid field: density 0, 1; density head 2; feature 3; colour 4 (with
// harmonics), 5; rgb head 6.
template <class T, class FE, class DE, class WS, class BP>
__device__ __forceinline__ void hash_field_forward(const FE& feats, const DE& sh, WS& ws, BP bias,
                                                   f32x16 (&sig)[T::SB], f32x16 (&rgb)[T::SB], int lane) {
    constexpr int K = NET_HASH_FIELD;
    constexpr int HS = out_steps<T, K, 0>();
    typename T::Op hA[HS][T::SB], hB[HS][T::SB];
    ws.begin();
    f32x16 b0 = load_bias16(bias, LayerInfo<T, K, 0>::bias, 0, lane >> 5);
    NoEpi none, none2;
    auto p0 = dense_layer<T, K, 0, 1>(feats, feats, hA, ws, bias, lane, b0, none);
    auto p1 = dense_layer<T, K, 1, 2>(hA, hA, hB, ws, bias, lane, b0, p0);
    dense_head<T, K, 2, 3>(hB, hB, sig, ws, bias, lane, b0, p1);
    auto p3 = dense_layer<T, K, 3, 4>(hB, hB, hA, ws, bias, lane, b0, none2);
    auto p4 = dense_layer<T, K, 4, 5>(hA, sh, hB, ws, bias, lane, b0, p3);
    auto p5 = dense_layer<T, K, 5, 6>(hB, hB, hA, ws, bias, lane, b0, p4);
    dense_head<T, K, 6, -1>(hA, hA, rgb, ws, bias, lane, b0, p5);
}

// ---------------------------------------------------------------------------
// Input operands
// ---------------------------------------------------------------------------

// Frequency encoding of (x0, x1, x2) with L frequencies, as value pairs:
// pair P = 3k + a (k < L) is (sin, cos) of 2^k x_a (times pi when use_pi),
// pair 3L is (x0, x1), pair 3L + 1 is (x2, 0), later pairs are zero.
struct PairSrc {
    int kind;  // 0 sin/cos, 1 (x0, x1), 2 (x2, 0), 3 zero
    int k, ax;
};
NERF_HD constexpr PairSrc pair_src(int P, int L) {
    return P < 3 * L ? PairSrc{0, P / 3, P % 3}
                     : (P == 3 * L ? PairSrc{1, 0, 0} : (P == 3 * L + 1 ? PairSrc{2, 0, 0} : PairSrc{3, 0, 0}));
}

// (sin, cos) of pi*arg (PI) or of arg.  With pi, arg/2 is a number of
// revolutions: removing its nearest integer is exact in float32, and the
// hardware sine and cosine take the remaining [-1/2, 1/2] revolution.
// Without pi the library's accurately reduced sincosf is used.
template <bool PI>
__device__ __forceinline__ void enc_sincos(float arg, float& s, float& c) {
    if constexpr (PI) {
        const float t = arg * 0.5f;
        const float r = t - rintf(t);
        s = __builtin_amdgcn_sinf(r);
        c = __builtin_amdgcn_cosf(r);
    } else {
        sincosf(arg, &s, &c);
    }
}

template <int KIND>
__device__ __forceinline__ void enc_plain(const float (&x)[3], float& a, float& b) {
    if constexpr (KIND == 1) {
        a = x[0];
        b = x[1];
    } else if constexpr (KIND == 2) {
        a = x[2];
        b = 0.0f;
    } else {
        a = 0.0f;
        b = 0.0f;
    }
}

// Pair P0 for lanes of half 0, P1 for half 1 (h = lane / 32): the argument
// is chosen per half first, so one sine/cosine serves both halves.
template <int P0, int P1, int L, bool PI>
__device__ __forceinline__ void enc_pair(int h, const float (&x)[3], float& a, float& b) {
    constexpr PairSrc s0 = pair_src(P0, L), s1 = pair_src(P1, L);
    if constexpr (s0.kind == 0 && s1.kind == 0) {
        const float arg = h ? x[s1.ax] * (float)(1 << s1.k) : x[s0.ax] * (float)(1 << s0.k);  // exact scaling
        enc_sincos<PI>(arg, a, b);
    } else if constexpr (s0.kind == 0 || s1.kind == 0) {
        constexpr PairSrc st = s0.kind == 0 ? s0 : s1, sp = s0.kind == 0 ? s1 : s0;
        float ta, tb, pa, pb;
        enc_sincos<PI>(x[st.ax] * (float)(1 << st.k), ta, tb);
        enc_plain<sp.kind>(x, pa, pb);
        const bool trig = (h != 0) == (s1.kind == 0);
        a = trig ? ta : pa;
        b = trig ? tb : pb;
    } else {
        float a0, b0, a1, b1;
        enc_plain<s0.kind>(x, a0, b0);
        enc_plain<s1.kind>(x, a1, b1);
        a = h ? a1 : a0;
        b = h ? b1 : b0;
    }
}

template <int L, bool PI, int NS>
__device__ __forceinline__ void enc_operands_t(bf16x8 (&enc)[NS][2], const float (&x)[2][3], int lane) {
    const int h = lane >> 5;
    static_for<0, NS>([&](auto s) {
        static_for<0, 2>([&](auto sb) {
            bf16x8 v;
            static_for<0, 4>([&](auto jp) {
                float a, b;
                enc_pair<8 * s.value + jp.value, 8 * s.value + 4 + jp.value, L, PI>(h, x[sb.value], a, b);
                v[2 * jp.value] = to_bf16(a);
                v[2 * jp.value + 1] = to_bf16(b);
            });
            enc[s.value][sb.value] = v;
        });
    });
}

template <int L, bool PI, int NS>
__device__ __forceinline__ void enc_operands_t(float (&enc)[NS][1], const float (&x)[1][3], int lane) {
    const int h = lane >> 5;
    static_for<0, NS / 2>([&](auto p) {
        float a, b;
        enc_pair<2 * p.value, 2 * p.value + 1, L, PI>(h, x[0], a, b);
        enc[2 * p.value][0] = a;
        enc[2 * p.value + 1][0] = b;
    });
}

// Operands of the encoded input for the packer's slot order.
template <int L, class Op, int NS, int SB>
__device__ __forceinline__ void enc_operands(Op (&enc)[NS][SB], const float (&x)[SB][3], bool use_pi, int lane) {
    if (use_pi)
        enc_operands_t<L, true>(enc, x, lane);
    else
        enc_operands_t<L, false>(enc, x, lane);
}

// Operands of a segment read from a row-major float32 matrix (`row[sb]`
// points at the sample's row), following the packer's slot order.
template <int NS>
__device__ __forceinline__ void row_operands(bf16x8 (&op)[NS][2], Seg seg, const float* const (&row)[2], int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            bf16x8 v;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // padding columns (c < 0) load column 0 and discard it, so
                // every load issues unconditionally and back to back
                const int c = seg_col(seg, PREC_BF16, s, h, j);
                const float x = row[sb][c >= 0 ? c : 0];
                v[j] = to_bf16(c >= 0 ? x : 0.0f);
            }
            op[s][sb] = v;
        }
}

template <int NS>
__device__ __forceinline__ void row_operands(float (&op)[NS][1], Seg seg, const float* const (&row)[1], int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int c = seg_col(seg, PREC_F32, s, h, 0);
        const float x = row[0][c >= 0 ? c : 0];
        op[s][0] = c >= 0 ? x : 0.0f;
    }
}

}  // namespace nerf
