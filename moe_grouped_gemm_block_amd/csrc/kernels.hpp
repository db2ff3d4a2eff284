// Which translation unit defines which kernels.
//
// Every kernel of the library is defined in exactly one translation unit and
// declared in all others, so that the kernels compile in parallel.  A
// translation unit that defines a group says so before including the kernel
// headers:
//   DG_DEFINE_FMT_44  E4M3 A x E4M3 B   (kernels without format suffix)
//   DG_DEFINE_FMT_45  E4M3 A x E5M2 B   (suffix _a4b5)
//   DG_DEFINE_FMT_54  E5M2 A x E4M3 B   (suffix _a5b4)
//   DG_DEFINE_FMT_55  E5M2 A x E5M2 B   (suffix _a5b5)
//   DG_DEFINE_MISC    the quantiser
// The kernel headers pass DG_KERNEL(<family>, <group>) as the macro that
// emits each kernel: <family>_DEF (definition) or <family>_DECL (declaration).
#pragma once

#define DG_CAT_(a, b) a##b
#define DG_CAT(a, b) DG_CAT_(a, b)

#ifdef DG_DEFINE_FMT_44
#define DG_MODE_FMT_44 _DEF
#else
#define DG_MODE_FMT_44 _DECL
#endif
#ifdef DG_DEFINE_FMT_45
#define DG_MODE_FMT_45 _DEF
#else
#define DG_MODE_FMT_45 _DECL
#endif
#ifdef DG_DEFINE_FMT_54
#define DG_MODE_FMT_54 _DEF
#else
#define DG_MODE_FMT_54 _DECL
#endif
#ifdef DG_DEFINE_FMT_55
#define DG_MODE_FMT_55 _DEF
#else
#define DG_MODE_FMT_55 _DECL
#endif
#ifdef DG_DEFINE_MISC
#define DG_MODE_MISC _DEF
#else
#define DG_MODE_MISC _DECL
#endif

#define DG_KERNEL(FAMILY, GROUP) DG_CAT(FAMILY, DG_CAT(DG_MODE_, GROUP))
