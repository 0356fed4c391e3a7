// One instantiation unit of the device kernels: compiled once per weight
// type (MK_WT_BF16 or MK_WT_F32) and batch tile MK_NB; MK_LDS_STREAM selects
// the batch-1 variant that streams weights through an LDS page ring, and
// MK_W4_KERNELS the batch >= 4 instances for 4-bit layer matrices.
#include "megakernel.h"
#include "kernels.h"

#if defined(MK_WT_BF16)
#define MK_WT mk::bf16_t
#define MK_TAG bf16
#elif defined(MK_WT_F32)
#define MK_WT float
#define MK_TAG f32
#else
#error "define MK_WT_BF16 or MK_WT_F32"
#endif
#ifndef MK_NB
#error "define MK_NB"
#endif

#define MK_CAT3(a, b, c) a##b##_##c
#define MK_CAT4(a, b, c, d) a##b##_##c##d
#ifdef MK_LDS_STREAM
#define MK_NAME(tag, nb) MK_CAT4(mk_kernels_, tag, nb, s)
#elif defined(MK_W4_KERNELS)
#define MK_NAME(tag, nb) MK_CAT4(mk_kernels_, tag, nb, w)
#else
#define MK_NAME(tag, nb) MK_CAT3(mk_kernels_, tag, nb)
#endif

extern "C" void* MK_NAME(MK_TAG, MK_NB)(int kind) {
    switch (kind) {
        case mk::KK_PERSISTENT: return (void*)mk::k_persistent<MK_WT, MK_NB>;
        case mk::KK_LEVEL_GEMV: return (void*)mk::k_level_gemv<MK_WT, MK_NB>;
        default: return (void*)mk::k_level_attn<MK_WT>;
    }
}
