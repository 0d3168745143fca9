// copy_chunk.h -- the wavefront chunk copy shared by the copy kernels
// (kvcopy_kernel.hip, device_batch.hip).  Device code only; include inside
// namespace kvc { namespace { ... } }.
#pragma once

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
#define KVC_GLOBAL __attribute__((address_space(1)))

// Raw buffer resources.  The fourth descriptor word is the gfx9-family raw
// buffer format (32-bit data format, no swizzle, no stride).  A buffer access
// at an offset at or beyond num_records is dropped (stores) or reads zero
// (loads); every vector access here is either wholly inside or wholly
// outside its range, so the lanes past the end of a short row need no exec
// masking.  Without per-row branches the compiler keeps all loads of a pass
// in flight and waits with vmcnt(N) before each store, never vmcnt(0).
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy: loads plain, stores nontemporal ("nt", bit 1 of the
// cache-policy operand on gfx940+).  Measured on MI355X for 65,536 random
// 4 KiB blocks between two 1 GiB device pools: with one call repeated, plain
// loads with nt stores move 6.1-6.5 TB/s of HBM traffic (the memory-side
// cache keeps most sources), against 4.7-4.9 TB/s with nt on both sides or
// on neither; with calls cycling over 8 different batches every combination
// tried lands at 4.7-5.0 TB/s and this one at the top.  For mapped host
// memory the combinations are within noise of each other.
constexpr int kLoadPolicy = 0;
constexpr int kStorePolicy = 2;
// The sc1 form: sc1 | nt (bits 4 and 1).  On the gfx940 family the two
// scope bits SC1:SC0 name the coherence scope of an access (0 wavefront, 1
// workgroup, 2 device, 3 system), so sc1 alone is a device-scope,
// nontemporal store.  D2H kernels and the one-launch pair store this way by
// default.  Measured on MI355X (16,384 x 4 KiB each way, 300 steps after
// 300 warm-up steps, three processes per setting in alternating order): H2D
// and D2H on two streams at 128 workgroups each move 94.2-94.6 GB/s with the
// D2H kernel's stores in this form and 87.9-88.4 GB/s with nt alone, whatever
// form the H2D kernel's stores take; a lone D2H batch moves 56.7 against
// 52.7 GB/s.  The nt form also wrote 65.66 MiB per 64 MiB D2H launch
// (FETCH/WRITE_SIZE counters), this one exactly 64.00 MiB.  H2D and D2D
// stores, which land in HBM, keep nt; KVCOPY_F_STORE_SC1 / KVCOPY_F_STORE_NT
// force one form.
constexpr int kSc1StorePolicy = 18;
constexpr uint32_t kRowBytes = 64u * 16u;          // one wavefront instruction: 1 KiB
constexpr int kMaxRows = 16;                       // 16 KiB per pass, 64 VGPRs of data
constexpr uint32_t kPassBytes = kRowBytes * kMaxRows;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(uint64_t base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), 0, (int)bytes,
                                             kRsrcWord3);
}

// R rows of 1 KiB: all loads first, then all stores (cache policy SP).
template <int R, int SP>
__device__ __forceinline__ void copy_rows(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rd,
                                          uint32_t voff)
{
    v4u v[R];
#pragma unroll
    for (int j = 0; j < R; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(voff + j * kRowBytes), 0,
                                                     kLoadPolicy);
#pragma unroll
    for (int j = 0; j < R; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(v[j], rd, (int)(voff + j * kRowBytes), 0, SP);
}

// One wavefront copies one chunk.  src, dst and bytes are wave-uniform.
template <int SP = kStorePolicy>
__device__ __forceinline__ void copy_chunk(uint64_t src, uint64_t dst, uint32_t bytes,
                                           uint32_t lane)
{
    const uint32_t body = bytes & ~15u;
    const uint32_t voff = lane * 16u;
    for (uint32_t off = 0; off < body; off += kPassBytes) {
        const uint32_t pb = body - off < kPassBytes ? body - off : kPassBytes;
        const __amdgpu_buffer_rsrc_t rs = rsrc(src + off, pb);
        const __amdgpu_buffer_rsrc_t rd = rsrc(dst + off, pb);
        switch ((pb + kRowBytes - 1) / kRowBytes) {
        case 1: copy_rows<1, SP>(rs, rd, voff); break;
        case 2: copy_rows<2, SP>(rs, rd, voff); break;
        case 3: copy_rows<3, SP>(rs, rd, voff); break;
        case 4: copy_rows<4, SP>(rs, rd, voff); break;
        case 5: copy_rows<5, SP>(rs, rd, voff); break;
        case 6: copy_rows<6, SP>(rs, rd, voff); break;
        case 7: copy_rows<7, SP>(rs, rd, voff); break;
        case 8: copy_rows<8, SP>(rs, rd, voff); break;
        case 9: copy_rows<9, SP>(rs, rd, voff); break;
        case 10: copy_rows<10, SP>(rs, rd, voff); break;
        case 11: copy_rows<11, SP>(rs, rd, voff); break;
        case 12: copy_rows<12, SP>(rs, rd, voff); break;
        case 13: copy_rows<13, SP>(rs, rd, voff); break;
        case 14: copy_rows<14, SP>(rs, rd, voff); break;
        case 15: copy_rows<15, SP>(rs, rd, voff); break;
        default: copy_rows<16, SP>(rs, rd, voff); break;
        }
    }
    if ((bytes & 8u) && lane == 0) {   // a range that ends in an odd 8-byte word
        const uint64_t w = *reinterpret_cast<KVC_GLOBAL const uint64_t *>(src + body);
        __builtin_nontemporal_store(w, reinterpret_cast<KVC_GLOBAL uint64_t *>(dst + body));
    }
}

