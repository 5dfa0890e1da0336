// The NF4 code table as fp32 literals, shared by the device kernels and the host ABI.
// 16 standard-normal quantile levels, ascending, with exact -1 (index 0), 0 (index 7)
// and +1 (index 15); the construction is stated in lnf4.h (lnf4_nf4_table).
#pragma once

#define LNF4_TABLE_INIT                                                                       \
  {-0x1p+0f,         -0x1.647362p-1f, -0x1.0cd65cp-1f, -0x1.94653cp-2f, -0x1.234496p-2f,     \
   -0x1.7a6a7ap-3f,  -0x1.74f0d2p-4f, 0.0f,            0x1.45f602p-4f,  0x1.4995bep-3f,      \
   0x1.f809b4p-3f,   0x1.5a066cp-2f,  0x1.c3496ap-2f,  0x1.200f52p-1f,  0x1.722760p-1f,      \
   0x1p+0f}
