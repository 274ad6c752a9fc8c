#include <hip/hip_runtime.h>
#include <stdint.h>
#define LDS __attribute__((address_space(3)))
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k(const uint16_t* a, float* out, int nsteps) {
  __shared__ __attribute__((aligned(16))) uint16_t s[4][8192];
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)a, 0, 0x7fffffff, 0x00020000);
  int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  f32x16_t acc = {};
  for (int st = 0; st < 3; ++st)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS void*)&s[st][w * 512], 16, l * 16, st * 4096, 0, 0);
  for (int st = 0; st < nsteps; ++st) {
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
    if (st + 3 < nsteps)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS void*)&s[(st + 3) & 3][w * 512], 16, l * 16, (st + 3) * 4096, 0, 0);
    const uint16_t* b = s[st & 3];
    bf16x8_t x = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(b + l * 8));
    bf16x8_t y = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(b + 512 + l * 8));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc, 0, 0, 0);
  }
  for (int i = 0; i < 16; ++i) out[threadIdx.x * 16 + i] = acc[i];
}
